// 2^y in float64 for the draws of the verifier's kernels (the residual, bonus and tree draws need weights to float64
// accuracy: a token boundary of the draw's CDF often lies within 1e-7 of the draw point at these vocabulary sizes).
//
// Table-driven in the manner of Tang's exponential (P. T. P. Tang, ACM TOMS 15(2), 1989): y is rounded to a multiple
// of 1/256, n = 256 k + j; 2^(j/256) comes from a 256-entry table in LDS, 2^f for the remainder |f| <= 1/512 from its
// degree-4 Taylor polynomial (truncation below 4e-17 relative) and 2^k is applied exactly with ldexp. Every workgroup
// that draws fills the table first (fexp_fill_table, one entry per thread of a 256-thread workgroup). The _at forms
// take the table's place in the caller's own LDS (a kernel that overlays it on other shared arrays).
#pragma once

#include <hip/hip_runtime.h>

namespace sv {
namespace {

__shared__ double s_exp2tab[256];

// By every thread of a 256-thread workgroup, before any fexp call (a barrier must follow before the first use).
__device__ __forceinline__ void fexp_fill_table_at(double* tab) {
  tab[threadIdx.x] = exp2(double(threadIdx.x) * 0.00390625);
}
__device__ __forceinline__ void fexp_fill_table() { fexp_fill_table_at(s_exp2tab); }

// The core takes a finite y in [-2000, 1023]; below -1075 its result is exactly 0 (ldexp underflows).
__device__ __forceinline__ double fexp_core_at(const double* tab, double y) {
  const double kMagic = 26388279066624.0;                      // 1.5 * 2^44: its ulp is 1/256
  const double t = y + kMagic;
  const int n = int(__double2loint(t));                        // round(256 y), two's complement in the low bits
  const double f = y - (t - kMagic);                           // y - n / 256, exact, |f| <= 1/512
  double q = fma(0x1.3b2ab6fba4e77p-7, f, 0x1.c6b08d704a0c0p-5);  // ln2^4/24, ln2^3/6
  q = fma(q, f, 0x1.ebfbdff82c58fp-3);                         // ln2^2/2
  q = fma(q, f, 0x1.62e42fefa39efp-1);                         // ln2
  q = fma(q, f, 1.0);
  return ldexp(tab[n & 255] * q, n >> 8);
}
__device__ __forceinline__ double fexp_core(double y) { return fexp_core_at(s_exp2tab, y); }

// Any y up to 1023: the argument is clamped at -2000 (one instruction), so -inf and every y below -1075 give exactly
// 0. NaN gives 0 too: a row holding NaN or +inf is reported as non-finite before any weight of it is used.
__device__ __forceinline__ double fexp_scaled_at(const double* tab, double y) {
  return fexp_core_at(tab, fmax(y, -2000.0));
}
__device__ __forceinline__ double fexp_scaled(double y) { return fexp_core(fmax(y, -2000.0)); }

// The exponent (z - m) * log2(e) / T of an element, formed as z * c2 + nm with one rounding, nm = -(m * c2). Every
// evaluation of an element's weight goes through here, so repeated evaluations agree bit for bit.
__device__ __forceinline__ double xarg(float z, double c2, double nm) { return fma(double(z), c2, nm); }

}  // namespace
}  // namespace sv
