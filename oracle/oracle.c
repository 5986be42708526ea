/*
 * oracle.c -- CPU oracle for the N-way tensor-parallel AllReduce sum.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker of the HIP
 * path.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py may load it.  It shares no code, header, table or constant with the
 * GPU library (message_allreduce_amd/csrc, include/llar.h); nothing on the
 * product path may call it.
 *
 * What it computes (plain definition, no blocking, no reordering):
 *
 *   "Every Microsecond Matters: Achieving Near Speed-of-Light Latency in GPU
 *   Collectives" (agihunt.info summary), section on why small AllReduces
 *   matter: each decode step combines the N tensor-parallel shard outputs of a
 *   layer with one AllReduce, i.e. out[i] = sum over ranks r of partial_r[i].
 *   Same page, paragraph "Two-shot LL128": the reduction is addition only and is
 *   defined for FP32, FP16 and BF16.
 *   yololab.net "parallelism vs network" page, collective table: All-Reduce
 *   leaves every rank holding the full reduced result.
 *
 * The pages say nothing about the order or precision of the additions, nor
 * about rounding.  Reading adopted here (plainest one):
 *   1. decode every element exactly to IEEE binary64;
 *   2. add in rank order, s = (((p0 + p1) + p2) + ... + p_{N-1}), in binary64,
 *      starting from p0 itself (so that -0 + -0 stays -0);
 *   3. round s once to the output type with round-to-nearest, ties-to-even,
 *      overflow to +-Inf, gradual underflow; NaN stays NaN (payload ignored).
 *
 * Rounding is written out from the IEEE 754 definition on the binary64 bit
 * pattern (sign, biased exponent, 52-bit fraction): keep the significand bits
 * down to the target quantum, compare the discarded part with one half
 * quantum, break an exact tie toward an even last kept bit.
 *
 * Build: gcc -O2 -fPIC -shared -o liboracle.so oracle.c  (plain C99).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

/* dtype codes used by this file's ABI (the Python wrapper in this directory
 * passes them): 0 = binary32, 1 = binary16, 2 = bfloat16. */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* IEEE format description: exponent field width and stored fraction width. */
typedef struct { int ebits; int mbits; } fmt_t;

static fmt_t fmt_of(int dtype) {
  fmt_t f;
  switch (dtype) {
    case OR_F32: f.ebits = 8; f.mbits = 23; break;
    case OR_F16: f.ebits = 5; f.mbits = 10; break;
    default:     f.ebits = 8; f.mbits = 7; break; /* bfloat16 */
  }
  return f;
}

static uint64_t bits_of_double(double x) { uint64_t u; memcpy(&u, &x, 8); return u; }

/* ---- decode: stored bit pattern -> exact binary64 value ------------------ */
/* value = (-1)^s * significand * 2^(exp - bias - mbits), where significand is
 * the stored fraction plus the hidden one for normal numbers; the exponent of a
 * subnormal is that of the smallest normal.  All three formats embed exactly in
 * binary64. */
double oracle_decode_bits(int dtype, uint32_t bits) {
  fmt_t f = fmt_of(dtype);
  int bias = (1 << (f.ebits - 1)) - 1;
  uint32_t sign = (bits >> (f.ebits + f.mbits)) & 1u;
  uint32_t e = (bits >> f.mbits) & ((1u << f.ebits) - 1u);
  uint32_t m = bits & ((1u << f.mbits) - 1u);
  double v;
  if (e == (1u << f.ebits) - 1u) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (e == 0) {
    v = ldexp((double)m, 1 - bias - f.mbits);
  } else {
    v = ldexp((double)(m | (1u << f.mbits)), (int)e - bias - f.mbits);
  }
  return sign ? -v : v;
}

/* ---- round: binary64 value -> nearest representable, ties to even -------- */
uint32_t oracle_round_bits(int dtype, double x) {
  fmt_t f = fmt_of(dtype);
  const int bias = (1 << (f.ebits - 1)) - 1;
  const int emin = 1 - bias;                 /* exponent of the smallest normal */
  const uint32_t sign = (uint32_t)(bits_of_double(x) >> 63) << (f.ebits + f.mbits);
  const uint32_t inf_bits = ((1u << f.ebits) - 1u) << f.mbits;

  uint64_t u = bits_of_double(x);
  int E = (int)((u >> 52) & 0x7FF);
  uint64_t M = u & ((1ull << 52) - 1ull);

  if (E == 0x7FF) {                          /* Inf or NaN */
    if (M == 0) return sign | inf_bits;
    return sign | inf_bits | (1u << (f.mbits - 1));   /* a quiet NaN */
  }
  if (E == 0) {
    /* zero, or a binary64 subnormal: below 2^-1022, far under half of the
     * smallest subnormal of every target format, so it rounds to a signed 0. */
    return sign;
  }
  int e = E - 1023;                          /* unbiased exponent of x */
  if (e > bias) return sign | inf_bits;      /* |x| >= 2^(emax+1): overflow */

  /* x = sig * 2^(e-52) with sig a 53-bit integer.  The target quantum is
   * 2^(max(e,emin) - mbits); d = number of low bits of sig below it. */
  uint64_t sig = M | (1ull << 52);
  int eq = (e < emin ? emin : e);
  int d = (52 - f.mbits) + (eq - e);
  uint64_t q;                                /* kept significand, in quanta */
  if (d >= 64) {
    q = 0;                                   /* less than a quarter quantum */
  } else {
    uint64_t rem = sig & ((1ull << d) - 1ull);
    uint64_t half = 1ull << (d - 1);
    q = sig >> d;
    if (rem > half || (rem == half && (q & 1ull))) q += 1;
  }
  /* Encode q quanta at exponent eq.  With the hidden bit counted inside q, a
   * normal result is ((eq + bias - 1) << mbits) + q; a subnormal (eq == emin,
   * q < 2^mbits) is q itself since eq + bias - 1 == 0; a carry out of the
   * significand moves into the exponent field by plain addition. */
  uint64_t enc = ((uint64_t)(eq + bias - 1) << f.mbits) + q;
  if (enc >= inf_bits) return sign | inf_bits;
  return sign | (uint32_t)enc;
}

/* ---- element access ------------------------------------------------------ */
static uint32_t load_bits(int dtype, const void* p, size_t i) {
  if (dtype == OR_F32) { uint32_t v; memcpy(&v, (const char*)p + 4 * i, 4); return v; }
  uint16_t h; memcpy(&h, (const char*)p + 2 * i, 2); return h;
}
static void store_bits(int dtype, void* p, size_t i, uint32_t v) {
  if (dtype == OR_F32) { memcpy((char*)p + 4 * i, &v, 4); return; }
  uint16_t h = (uint16_t)v; memcpy((char*)p + 2 * i, &h, 2);
}

/* out[i] = RNE_T( ((p0[i] + p1[i]) + ...) + p_{N-1}[i] ), sums in binary64.
 * partials: n_ranks host pointers to n elements each; out: n elements.
 * Returns 0, or -1 on a bad argument. */
int oracle_allreduce(const void* const* partials, int n_ranks, size_t n, int dtype, void* out) {
  if (n_ranks < 1 || !partials || (!out && n) || dtype < 0 || dtype > 2) return -1;
  for (size_t i = 0; i < n; ++i) {
    double s = oracle_decode_bits(dtype, load_bits(dtype, partials[0], i));
    for (int r = 1; r < n_ranks; ++r) s += oracle_decode_bits(dtype, load_bits(dtype, partials[r], i));
    store_bits(dtype, out, i, oracle_round_bits(dtype, s));
  }
  return 0;
}

/* The binary64 sum alone (before rounding), for tests of the error bound of
 * the non-deterministic atomic protocol. */
int oracle_sum_f64(const void* const* partials, int n_ranks, size_t n, int dtype, double* out) {
  if (n_ranks < 1 || !partials || (!out && n) || dtype < 0 || dtype > 2) return -1;
  for (size_t i = 0; i < n; ++i) {
    double s = oracle_decode_bits(dtype, load_bits(dtype, partials[0], i));
    for (int r = 1; r < n_ranks; ++r) s += oracle_decode_bits(dtype, load_bits(dtype, partials[r], i));
    out[i] = s;
  }
  return 0;
}

/* Vector forms of decode/round for the tests. */
void oracle_decode_array(int dtype, const void* src, size_t n, double* dst) {
  for (size_t i = 0; i < n; ++i) dst[i] = oracle_decode_bits(dtype, load_bits(dtype, src, i));
}
void oracle_round_array(int dtype, const double* src, size_t n, void* dst) {
  for (size_t i = 0; i < n; ++i) store_bits(dtype, dst, i, oracle_round_bits(dtype, src[i]));
}
