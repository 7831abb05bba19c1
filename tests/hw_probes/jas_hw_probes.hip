// jas_hw_probes.hip -- test-only probes of gfx950 instructions the library
// relies on.  Not part of the library; built beside the tests.
//
//  * exp2 sweep: every negative binary32 u (down to -inf) through v_exp_f32, against
//    2^u evaluated in double and rounded to binary32 with results below
//    2^-126 taken as +0 (the library's exponential contract).  Reports the
//    largest difference in ulps and every place where the flush behaviour
//    differs.
//  * bf16 conversion sweep: every binary32 bit pattern through
//    v_cvt_pk_bf16_f32 against round-to-nearest-even on the bit pattern.
//  * fp16 conversion sweep: every binary32 bit pattern through the packed
//    binary32 -> binary16 conversion against round-to-nearest-even
//    (subnormals kept, overflow to infinity).
//  * log2 sweep: every binary32 in [1, 2^18 + 1] (the range of a row's sum L
//    for rows of up to 262,144 keys and a sink) through v_log_f32 against
//    log2 in double rounded to binary32.
//  * copy16 / read2_write1: 16-byte streams (one read and one write, two
//    reads and one write per word), the attainable HBM rates of the
//    softmax forward's and backward's access mixes, and the calibration
//    point of the HBM byte counters.
//  * transposed LDS read (ds_read_b64_tr_b16) lane layout: which 16-bit
//    elements each lane receives for given per-lane addresses.
//  * MFMA operand layout: one 16x16x32 bf16 / fp16 product with the operands
//    placed by the layout the attention kernel assumes (A: lane = row +
//    16*(k/8), element k%8; B: lane = col + 16*(k/8), element k%8; D: lane =
//    col + 16*(row/4), element row%4).
//
// Each thread handles kPer consecutive inputs; each workgroup writes its own
// four result words, no atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
constexpr int kThreads = 256;
constexpr int kPer = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ inline float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ inline uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ inline uint32_t ord(float f) {  // monotone map of finite floats to integers
  uint32_t u = f2u(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// out[4*block + 0] = max |ulp diff|, +1 = #u with diff != 0,
// +2 = #u >= -126 whose result is below 2^-126, +3 = #u < -126 whose result is not +0
__global__ void exp2_sweep(uint32_t first, uint32_t count, uint32_t *out) {
  uint32_t mx = 0, ndiff = 0, nlow = 0, nnz = 0;
  const uint32_t base = (blockIdx.x * kThreads + threadIdx.x) * kPer;
  for (int i = 0; i < kPer; ++i) {
    const uint32_t k = base + i;
    if (k >= count) break;
    const float u = u2f(first + k);  // negative floats: bit patterns increase toward -inf
    const float hw = __builtin_amdgcn_exp2f(u);
    float ref;
    if (u < -126.0f) ref = 0.0f;
    else ref = (float)exp2((double)u);
    const uint32_t a = ord(hw), b = ord(ref);
    const uint32_t d = a > b ? a - b : b - a;
    mx = d > mx ? d : mx;
    ndiff += d != 0;
    if (u >= -126.0f && !(hw >= 0x1p-126f)) ++nlow;
    if (u < -126.0f && f2u(hw) != 0u) ++nnz;
  }
  __shared__ uint32_t s[4][kThreads];
  s[0][threadIdx.x] = mx; s[1][threadIdx.x] = ndiff; s[2][threadIdx.x] = nlow; s[3][threadIdx.x] = nnz;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r0 = 0, r1 = 0, r2 = 0, r3 = 0;
    for (int t = 0; t < kThreads; ++t) {
      r0 = s[0][t] > r0 ? s[0][t] : r0; r1 += s[1][t]; r2 += s[2][t]; r3 += s[3][t];
    }
    out[4 * blockIdx.x + 0] = r0; out[4 * blockIdx.x + 1] = r1;
    out[4 * blockIdx.x + 2] = r2; out[4 * blockIdx.x + 3] = r3;
  }
}

__device__ inline uint32_t rne_bits(uint32_t u) {
  uint32_t lo = u >> 16, rest = u & 0xffffu;
  if (rest > 0x8000u || (rest == 0x8000u && (lo & 1u))) lo += 1u;
  return lo;
}

// out[2*block + 0] = #non-NaN patterns whose conversion differs from RNE,
// +1 = #NaN patterns whose result is not a NaN
__global__ void bf16_sweep(uint64_t first, uint64_t count, uint32_t *out) {
  uint32_t bad = 0, badnan = 0;
  const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
  for (int i = 0; i < kPer; i += 2) {
    const uint64_t k = base + i;
    if (k >= count) break;
    const uint32_t u0 = (uint32_t)(first + k), u1 = (uint32_t)(first + k + 1);
    f32x2_t v = {u2f(u0), u2f(u1)};
    const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    const uint32_t h[2] = {w & 0xffffu, w >> 16};
    const uint32_t in[2] = {u0, u1};
    for (int j = 0; j < 2; ++j) {
      const bool isnan = (in[j] & 0x7f800000u) == 0x7f800000u && (in[j] & 0x7fffffu);
      if (isnan) badnan += !((h[j] & 0x7f80u) == 0x7f80u && (h[j] & 0x7fu));
      else bad += h[j] != rne_bits(in[j]);
    }
  }
  __shared__ uint32_t s[2][kThreads];
  s[0][threadIdx.x] = bad; s[1][threadIdx.x] = badnan;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r0 = 0, r1 = 0;
    for (int t = 0; t < kThreads; ++t) { r0 += s[0][t]; r1 += s[1][t]; }
    out[2 * blockIdx.x] = r0; out[2 * blockIdx.x + 1] = r1;
  }
}

// binary32 bits -> binary16 bits, round to nearest-even (not for NaN): the
// magnitude counted in binary16 units, 2^-24 below 2^-14 and 2^(E-10) above
// (E the unbiased exponent), the dropped bits deciding the rounding.
__device__ inline uint32_t f16_rne_ref(uint32_t u) {
  const uint32_t sign = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
  if (a >= 0x477ff000u) return sign | 0x7c00u;  // from 65520 up: infinity
  const uint32_t e = a >> 23;
  if (e < 102) return sign;                       // below 2^-25
  const uint32_t m = (a & 0x7fffffu) | 0x800000u;
  const uint32_t sh = (e >= 113) ? 13u : 126u - e;
  uint32_t q = m >> sh;
  const uint32_t rest = m & ((1u << sh) - 1u), half = 1u << (sh - 1u);
  if (rest > half || (rest == half && (q & 1u))) ++q;
  return (e >= 113) ? (sign | (((e - 113u) << 10) + q)) : (sign | q);
}

// out[2*block + 0] = #non-NaN patterns whose conversion differs from RNE,
// +1 = #NaN patterns whose result is not a NaN
__global__ void f16_sweep(uint64_t first, uint64_t count, uint32_t *out) {
  uint32_t bad = 0, badnan = 0;
  const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
  for (int i = 0; i < kPer; i += 2) {
    const uint64_t k = base + i;
    if (k >= count) break;
    const uint32_t u0 = (uint32_t)(first + k), u1 = (uint32_t)(first + k + 1);
    f32x2_t v = {u2f(u0), u2f(u1)};
    const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    const uint32_t h[2] = {w & 0xffffu, w >> 16};
    const uint32_t in[2] = {u0, u1};
    for (int j = 0; j < 2; ++j) {
      const bool isnan = (in[j] & 0x7f800000u) == 0x7f800000u && (in[j] & 0x7fffffu);
      if (isnan) badnan += !((h[j] & 0x7c00u) == 0x7c00u && (h[j] & 0x3ffu));
      else bad += h[j] != f16_rne_ref(in[j]);
    }
  }
  __shared__ uint32_t s[2][kThreads];
  s[0][threadIdx.x] = bad; s[1][threadIdx.x] = badnan;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r0 = 0, r1 = 0;
    for (int t = 0; t < kThreads; ++t) { r0 += s[0][t]; r1 += s[1][t]; }
    out[2 * blockIdx.x] = r0; out[2 * blockIdx.x + 1] = r1;
  }
}

// out[2*block + 0] = max |ulp diff| of v_log_f32 against log2 in double
// rounded to binary32, +1 = #inputs that differ
__global__ void log2_sweep(uint32_t first, uint32_t count, uint32_t *out) {
  uint32_t mx = 0, nd = 0;
  const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer;
  for (int i = 0; i < kPer; ++i) {
    const uint64_t k = base + i;
    if (k >= count) break;
    const float x = u2f((uint32_t)(first + k));
    const float hw = __builtin_amdgcn_logf(x);
    const float ref = (float)log2((double)x);
    const uint32_t a = ord(hw), b = ord(ref);
    const uint32_t d = a > b ? a - b : b - a;
    mx = d > mx ? d : mx;
    nd += d != 0;
  }
  __shared__ uint32_t s[2][kThreads];
  s[0][threadIdx.x] = mx; s[1][threadIdx.x] = nd;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r0 = 0, r1 = 0;
    for (int t = 0; t < kThreads; ++t) { r0 = s[0][t] > r0 ? s[0][t] : r0; r1 += s[1][t]; }
    out[2 * blockIdx.x] = r0; out[2 * blockIdx.x + 1] = r1;
  }
}

// A: 16x32 row-major, B: 32x16 row-major (16-bit patterns), D: 16x16 fp32.
// One wave.
__global__ void mfma_layout(const uint16_t *A, const uint16_t *B, float *D, int f16) {
  const int l = threadIdx.x & 63;
  const int rc = l % 16, kg = l / 16;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (f16) {
    f16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = __builtin_bit_cast(_Float16, A[rc * 32 + kg * 8 + i]);
      b[i] = __builtin_bit_cast(_Float16, B[(kg * 8 + i) * 16 + rc]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
  } else {
    bf16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = __builtin_bit_cast(__bf16, A[rc * 32 + kg * 8 + i]);
      b[i] = __builtin_bit_cast(__bf16, B[(kg * 8 + i) * 16 + rc]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  for (int r = 0; r < 4; ++r) D[(kg * 4 + r) * 16 + rc] = acc[r];
}

// Plain copy of n16 16-byte words: each thread moves 4 words per trip, all
// four loads issued before the stores; grid-stride over the buffer.  A
// bandwidth ceiling for kernels that read and write once, and a calibration
// point for the HBM byte counters.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(256) void copy16(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                              uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * 256 * 4;
  for (uint64_t base = (uint64_t)blockIdx.x * 256 * 4 + threadIdx.x; base < n16; base += stride) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t k = base + (uint64_t)i * 256;
      if (k < n16) v[i] = NT ? __builtin_nontemporal_load(src + k) : src[k];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t k = base + (uint64_t)i * 256;
      if (k < n16) {
        if (NT) __builtin_nontemporal_store(v[i], dst + k);
        else dst[k] = v[i];
      }
    }
  }
}

// lane layout of gfx950's transposed LDS read ds_read_b64_tr_b16: LDS holds
// each 16-bit element's own index; lane l reads at element addr[l] (a
// multiple of 4, checked on the host to lie inside the array) and writes
// the 4 values it receives to out[4l .. 4l+3]
typedef short v4i16 __attribute__((ext_vector_type(4)));
constexpr int kTrElems = 8192;  // 16 KB: 32 rows of the attention kernel's V stride fit
__global__ void tr16_layout(const int *addr, uint16_t *out) {
  __shared__ __align__(16) uint16_t lds[kTrElems];
  for (int i = threadIdx.x; i < kTrElems; i += 64) lds[i] = (uint16_t)i;
  __syncthreads();
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(lds + addr[threadIdx.x]));
  for (int e = 0; e < 4; ++e) out[4 * threadIdx.x + e] = (uint16_t)r[e];
}

// lane layout of the gfx950 permlane swaps: out[2*lane], out[2*lane+1]
__global__ void permlane_layout(uint32_t *out) {
  const uint32_t l = threadIdx.x;
  auto p16 = __builtin_amdgcn_permlane16_swap(l, l, false, false);
  auto p32 = __builtin_amdgcn_permlane32_swap(l, l, false, false);
  out[4 * l + 0] = p16[0]; out[4 * l + 1] = p16[1];
  out[4 * l + 2] = p32[0]; out[4 * l + 3] = p32[1];
}
}  // namespace

// Two 16-byte reads (a and b) and one write (d) per word: the access mix
// of the softmax backward (P and dP read, dS written), in the shape of
// copy16 (4 words per thread per trip, every load before the stores).  The
// attainable rate of that mix on this machine, beside copy16's for the forward.
template <bool NT>
__global__ __launch_bounds__(256) void read2_write1(const u32x4 *__restrict__ a,
                                                    const u32x4 *__restrict__ b,
                                                    u32x4 *__restrict__ d, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * 256 * 4;
  for (uint64_t base = (uint64_t)blockIdx.x * 256 * 4 + threadIdx.x; base < n16; base += stride) {
    u32x4 x[4], y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t k = base + (uint64_t)i * 256;
      if (k < n16) {
        x[i] = NT ? __builtin_nontemporal_load(a + k) : a[k];
        y[i] = NT ? __builtin_nontemporal_load(b + k) : b[k];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t k = base + (uint64_t)i * 256;
      if (k < n16) {
        if (NT) __builtin_nontemporal_store(x[i] ^ y[i], d + k);
        else d[k] = x[i] ^ y[i];
      }
    }
  }
}

extern "C" {
// Sweep [first, first+count) (negative binary32 bit patterns).  out holds
// 4 words per workgroup; returns the number of workgroups used, or -1.
int probe_exp2_sweep(uint32_t first, uint32_t count, uint32_t *out, uint32_t out_words) {
  const uint64_t per_block = (uint64_t)kThreads * kPer;
  const uint64_t blocks = (count + per_block - 1) / per_block;
  if (blocks * 4 > out_words || blocks == 0) return -1;
  hipLaunchKernelGGL(exp2_sweep, dim3((unsigned)blocks), dim3(kThreads), 0, 0, first, count, out);
  return hipDeviceSynchronize() == hipSuccess ? (int)blocks : -1;
}

int probe_bf16_sweep(uint64_t first, uint64_t count, uint32_t *out, uint32_t out_words) {
  const uint64_t per_block = (uint64_t)kThreads * kPer;
  if (count % 2) return -1;
  const uint64_t blocks = (count + per_block - 1) / per_block;
  if (blocks * 2 > out_words || blocks == 0) return -1;
  hipLaunchKernelGGL(bf16_sweep, dim3((unsigned)blocks), dim3(kThreads), 0, 0, first, count, out);
  return hipDeviceSynchronize() == hipSuccess ? (int)blocks : -1;
}

int probe_f16_sweep(uint64_t first, uint64_t count, uint32_t *out, uint32_t out_words) {
  const uint64_t per_block = (uint64_t)kThreads * kPer;
  if (count % 2) return -1;
  const uint64_t blocks = (count + per_block - 1) / per_block;
  if (blocks * 2 > out_words || blocks == 0) return -1;
  hipLaunchKernelGGL(f16_sweep, dim3((unsigned)blocks), dim3(kThreads), 0, 0, first, count, out);
  return hipDeviceSynchronize() == hipSuccess ? (int)blocks : -1;
}

int probe_log2_sweep(uint32_t first, uint32_t count, uint32_t *out, uint32_t out_words) {
  const uint64_t per_block = (uint64_t)kThreads * kPer;
  const uint64_t blocks = (count + per_block - 1) / per_block;
  if (blocks * 2 > out_words || blocks == 0) return -1;
  hipLaunchKernelGGL(log2_sweep, dim3((unsigned)blocks), dim3(kThreads), 0, 0, first, count, out);
  return hipDeviceSynchronize() == hipSuccess ? (int)blocks : -1;
}

// Enqueue one copy of n16 16-byte words on `stream` (no synchronisation);
// blocks = 0 picks 4 workgroups per CU-ish (2048).  Returns 0 or -1.
int probe_copy16(const void *src, void *dst, uint64_t n16, int nontemporal, int blocks,
                 void *stream) {
  if (!src || !dst || ((uintptr_t)src | (uintptr_t)dst) % 16) return -1;
  const unsigned g = blocks > 0 ? (unsigned)blocks : 2048u;
  if (nontemporal)
    hipLaunchKernelGGL(copy16<true>, dim3(g), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)src, (u32x4 *)dst, n16);
  else
    hipLaunchKernelGGL(copy16<false>, dim3(g), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)src, (u32x4 *)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// A: 512 16-bit words, B: 512, D: 256 floats (device).
int probe_mfma_layout(const uint16_t *A, const uint16_t *B, float *D, int f16) {
  hipLaunchKernelGGL(mfma_layout, dim3(1), dim3(64), 0, 0, A, B, D, f16);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}

// addr: 64 host ints (element indices), out: 256 device 16-bit words.
// Returns -1 without launching when an address is not 8-byte aligned or
// would read past the 8192-element array.
int probe_tr16_layout(const int *addr_host, uint16_t *out) {
  for (int l = 0; l < 64; ++l)
    if (addr_host[l] < 0 || addr_host[l] % 4 != 0 || addr_host[l] + 4 > kTrElems) return -1;
  int *d = nullptr;
  if (hipMalloc(&d, 64 * sizeof(int)) != hipSuccess) return -1;
  if (hipMemcpy(d, addr_host, 64 * sizeof(int), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(d);
    return -1;
  }
  hipLaunchKernelGGL(tr16_layout, dim3(1), dim3(64), 0, 0, d, out);
  const hipError_t e = hipDeviceSynchronize();
  (void)hipFree(d);
  return e == hipSuccess ? 0 : -1;
}

int probe_permlane_layout(uint32_t *out) {  // out: 256 words
  hipLaunchKernelGGL(permlane_layout, dim3(1), dim3(64), 0, 0, out);
  return hipDeviceSynchronize() == hipSuccess ? 0 : -1;
}

// Enqueue one pass of read2_write1 over n16 16-byte words of a, b and d
// (16-byte aligned, d distinct from a and b) on `stream`; blocks = 0 picks
// 2048.  Returns 0 or -1.
int probe_read2_write1(const void *a, const void *b, void *d, uint64_t n16, int nontemporal,
                       int blocks, void *stream) {
  if (!a || !b || !d || ((uintptr_t)a | (uintptr_t)b | (uintptr_t)d) % 16) return -1;
  const unsigned g = blocks > 0 ? (unsigned)blocks : 2048u;
  if (nontemporal)
    hipLaunchKernelGGL(read2_write1<true>, dim3(g), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)a, (const u32x4 *)b, (u32x4 *)d, n16);
  else
    hipLaunchKernelGGL(read2_write1<false>, dim3(g), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)a, (const u32x4 *)b, (u32x4 *)d, n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
}
