// jas_launch.hip -- the per-head d_sink kernel, the compiled launch
// geometries and the dispatch of the row kernels by element type.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "jas.h"
#include "jas_kernels.h"

namespace jas {
namespace {

// ---------------------------------------------------------------------------
// d_sink: per head, 256-row chunks in (batch, query) order, balanced tree per
// chunk, chunk sums folded left to right.  One workgroup per head, one
// wavefront per chunk; lane l holds the chunk's rows 4l..4l+3.
// ---------------------------------------------------------------------------

constexpr int kDsinkWaves = 16;

__global__ __launch_bounds__(kWave * kDsinkWaves) void dsink_kernel(const DsinkArgs a) {
  __shared__ float part[kDsinkWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t h = blockIdx.x;
  const int64_t n = a.B * a.Sq;
  const int64_t chunks = (n + kTile - 1) / kTile;
  float D = 0.0f;
  for (int64_t k0 = 0; k0 < chunks; k0 += kDsinkWaves) {
    const int64_t k = k0 + wave;
    float cs = 0.0f;
    if (k < chunks) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t idx = k * kTile + lane * 4 + i;  // position in the head's row list
        if (idx < n) {
          const int64_t bb = idx / a.Sq, qq = idx - bb * a.Sq;
          v[i] = a.v[(bb * a.H + h) * a.Sq + qq];
        } else {
          v[i] = 0.0f;
        }
      }
      cs = group64_sum((v[0] + v[1]) + (v[2] + v[3]));
    }
    if (lane == 0) part[wave] = cs;
    __syncthreads();
    if (threadIdx.x == 0) {
      const int64_t m = (chunks - k0 < kDsinkWaves) ? chunks - k0 : kDsinkWaves;
      for (int64_t i = 0; i < m; ++i) D = (k0 + i == 0) ? part[i] : D + part[i];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) a.d_sink[h] = D;
}

}  // namespace

const int *compiled_cpls(int dtype, int *count) {
  if (dtype != 0) {  // 16-bit types
    *count = (int)(sizeof(kCplBf16) / sizeof(int));
    return kCplBf16;
  }
  *count = (int)(sizeof(kCplF32) / sizeof(int));
  return kCplF32;
}

bool cpl_compiled(int dtype, int wpr, int cpl) {
  if (wpr != 1 && wpr != 2 && wpr != 4) return false;
  int n = 0;
  const int *c = compiled_cpls(dtype, &n);
  for (int i = 0; i < n; ++i)
    if (c[i] == cpl) return true;
  return false;
}

bool stream_cpl_compiled(int dtype, int cpl) {
  const int *c = dtype == 0 ? kStreamCplF32 : kStreamCplBf16;
  return cpl == c[0] || cpl == c[1];
}

// Streaming segments of 64 tiles (16,384 keys): 4 waves x 8 slots for the
// 16-bit types, 4 x 16 for fp32.
int default_stream_cpl(int dtype) { return dtype == 0 ? kStreamCplF32[1] : kStreamCplBf16[1]; }

// Waves of a streaming workgroup.  The 16-bit backward takes 8 when the row
// fits in two segments of the wide workgroup (8 waves x 8 chunks per lane:
// 32,768 keys each): the last segment's P and dP stay in registers, the
// first segment's P in the LDS stash, and only that segment's dP is read
// twice (65,536-key rows: 0.572 ms against 0.646 ms with 4 waves, HBM bytes
// 1.17 instead of 1.30 times the algorithmic ones).  Every other streaming
// row takes 4 waves, whose segments of 16,384 keys let the last two stay in
// registers and the one before them wait in LDS: the forward is faster so
// (65,536 keys: 0.400 ms against 0.485 ms with 8 waves, whose two segments
// both stay in registers but at 170 VGPRs leave one workgroup per CU), and
// fp32 chunks in two register sets would not fit the wide workgroup's
// registers at four waves per SIMD.
int default_stream_wpr(int dtype, int nslots, bool backward) {
  if (dtype == 0 || !backward) return kBlockWaves;
  return nslots <= 2 * kStreamWideWaves * default_stream_cpl(dtype) ? kStreamWideWaves : kBlockWaves;
}

// Default waves per row for a row of `nslots` wave-wide chunks (the
// chunks-per-lane size then is the smallest compiled one that covers the
// row), and rows per workgroup.  Measured on MI355X, 16,384 rows of N keys,
// median of 5 x 20 calls over rotated copies; any choice gives the same
// bits.
//   16-bit forward (fp16 is laid out as bf16): one wavefront per row up to 5
//   slots (2,560 keys), two up to 18, four beyond.  At 6 to 9 slots two
//   wavefronts with two rows per workgroup take 3-12% less time than one
//   (4,352 keys: 48.9 us against 51.4), at 2 and 3 slots 15-25% more; on the
//   joint shape with its mask the two are level.
//   16-bit backward, which keeps two inputs in registers: one wavefront up to
//   4 slots, four beyond (two are within 1-2.5% from 5 to 8 slots).
//   fp32 (a slot is 256 keys): one wavefront up to 3 slots (backward: 2),
//   two up to 8, four beyond.  Against the earlier table (one wavefront per
//   row up to 17 slots forward and 8 backward) the forward takes 5-7% less
//   time from 4 slots up (1,024 keys: 23.5 us against 25.3; 4,352 keys: 92.7
//   us against 98.4) and the backward 4-9% less from 3 to 8 slots (2,048
//   keys: 63.0 us against 69.1, two rows per workgroup).
// Each threshold is capped at what the compiled chunk sizes cover (17 per
// lane for fp32), so every row up to 16,384 keys has a geometry.
int default_wpr(int dtype, int nslots, bool backward) {
  int n = 0;
  const int *c = compiled_cpls(dtype, &n);
  const int top = c[n - 1];  // largest compiled chunks per lane
  if (nslots > 4 * top) return 0;
  if (dtype == 0) return nslots <= (backward ? 2 : 3) ? 1 : nslots <= std::min(8, 2 * top) ? 2 : 4;
  if (backward) return nslots <= 4 ? 1 : 4;
  if (nslots <= std::min(5, top)) return 1;
  if (nslots <= std::min(18, 2 * top)) return 2;
  return 4;
}

// Default rows per workgroup for a row spread over `wpr` wavefronts: one row
// per wavefront, 4 rows per workgroup; a 16-bit forward row of up to 9 slots
// on two wavefronts, 2 rows (the 4,352-key rows: 48.4 us against 50.6 us
// for one row per workgroup, and the joint shape with its mask unchanged);
// an fp32 backward row on two wavefronts, 2 rows (2,048 keys: 63.0 us
// against 66.4); any other row spread over several wavefronts, one row per
// workgroup (measured faster: its barriers then couple only the row's own
// waves; 8,192 keys on two wavefronts: 1.38 ms against 1.51 ms with two
// rows).
int default_rpb(int dtype, int nslots, int wpr, bool backward) {
  if (wpr == 1) return kBlockWaves;
  if (wpr == 2 && !backward && dtype != 0 && nslots <= 9) return 2;
  if (wpr == 2 && backward && dtype == 0) return 2;
  return 1;
}

hipError_t launch_fwd(int dtype, const FwdArgs &a, const Geometry &g, hipStream_t st) {
  switch (dtype) {
    case 0: return launch_fwd_f32(a, g, st);
    case 1: return launch_fwd_bf16(a, g, st);
    case 2: return launch_fwd_f16(a, g, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(int dtype, const BwdArgs &a, const Geometry &g, hipStream_t st) {
  switch (dtype) {
    case 0: return launch_bwd_f32(a, g, st);
    case 1: return launch_bwd_bf16(a, g, st);
    case 2: return launch_bwd_f16(a, g, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dsink(const DsinkArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(dsink_kernel, dim3((unsigned)a.H), dim3(kWave * kDsinkWaves), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The library's own device scratch for jas_bwd_noalloc: the per-row d_sink
// shares of up to JAS_NOALLOC_MAX_ROWS rows (4 MiB), in the module's static
// device memory, so that the call allocates nothing.  Every GPU the library
// runs on holds its own copy at its own address until the process ends.  In
// host code `scratch` only names a host-side stand-in for the symbol; the
// device address is looked up once per device, with that device current,
// and only that address is handed to kernels.  The backward kernel writes
// every row's share before the d_sink kernel reads it, so nothing in it has
// to start at zero; calls on one GPU share it, so calls that overlap on one
// GPU (concurrent streams) race.
// ---------------------------------------------------------------------------

namespace {
constexpr int kScratchDevices = 64;
static __device__ __align__(256) float scratch[JAS_NOALLOC_MAX_ROWS];
std::mutex scratch_mu;
float *scratch_ptr[kScratchDevices];  // device address of `scratch`, per device; null until looked up
}  // namespace

hipError_t scratch_address(int device, float **out) {
  *out = nullptr;
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[device] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[device] = static_cast<float *>(p);
  }
  *out = scratch_ptr[device];
  return hipSuccess;
}

}  // namespace jas
