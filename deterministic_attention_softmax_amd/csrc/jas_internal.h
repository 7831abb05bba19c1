// Internal interface between the host validation layer (jas_api.cpp) and the
// gfx950 kernels (jas_kernels.h, instantiated per element type in
// jas_kernels_<dtype>.hip; jas_launch.hip dispatches).  Not installed; the public ABI is jas.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace jas {

constexpr int kTile = 256;         // keys per tile (fixed, never tuned)
constexpr int kWave = 64;          // CDNA wavefront
constexpr int kMaxKeys = 16384;              // longest row of the one-pass kernels
constexpr int kMaxTiles = kMaxKeys / kTile;  // 64: one tile state per lane
constexpr int kMaxStreamKeys = 262144;       // longest row of the streaming kernels
constexpr int kBlockWaves = 4;     // waves per workgroup (256 threads)
constexpr int kStreamWideWaves = 8;  // the wide streaming workgroup: one row on 512 threads

struct RowShape {
  int64_t rows;   // batch * heads * q_rows
  int64_t N;      // keys
  int64_t ld;     // row stride in elements
  int64_t H, Sq;  // for decoding row -> (b, h, q)
  int T;          // tiles per row
};

// Visible key prefix of a row: causal cut and per-batch key length.
struct Exclusion {
  int causal;              // key <= N - Sq + q
  const int32_t *key_len;  // [B] or nullptr
};

struct FwdArgs {
  const void *scores;
  void *probs;
  const float *mask;  // nullptr when no mask
  int64_t msb, msh, msq;
  Exclusion ex;
  const float *sink;  // nullptr when no sink
  float *p_sink;
  float *lse;         // nullptr when the row log-sum-exp is not asked for
  RowShape s;
  int vec_io;         // 16-byte path: rows (and mask rows) are whole aligned 16-byte chunks
  int vec_mask;       // mask rows start on 16-byte boundaries (or no mask)
  int stash;          // streaming kernels: segments kept in LDS (set by the launcher)
};

struct BwdArgs {
  const void *probs;
  const void *dprobs;
  void *dscores;
  const float *p_sink;  // nullptr when no sink
  float *v;             // per-row d_sink share (workspace), nullptr when no sink
  Exclusion ex;
  RowShape s;
  int vec_io;         // 16-byte path: rows are whole aligned 16-byte chunks
  int stash;          // streaming kernel: segments whose P is kept in LDS (set by the launcher)
};

struct DsinkArgs {
  const float *v;
  float *d_sink;
  int64_t B, H, Sq;
};

struct Geometry {
  int wpr;         // waves per row
  int cpl;         // 16-byte chunks per lane (compiled size); streaming: per segment
  int rpb;         // rows per workgroup
  int64_t blocks;  // grid size
  int stream;      // 1: the streaming kernels (4 waves per row, rows in segments)
  int mres;        // 1: forward with the mask kept in registers over runs of rows
};

// dtype codes: 0 fp32, 1 bf16, 2 fp16 (jas_dtype_t)
// Keys held by one 16-byte chunk: 8 bf16 / fp16 or 4 fp32.
inline int keys_per_chunk(int dtype) { return dtype == 0 ? 4 : 8; }
// Tiles covered by one wave-wide chunk (64 lanes x 16 bytes).
inline int tiles_per_slot(int dtype) { return dtype == 0 ? 1 : 2; }

bool cpl_compiled(int dtype, int wpr, int cpl);
int default_wpr(int dtype, int nslots, bool backward);
int default_rpb(int dtype, int nslots, int wpr, bool backward);
const int *compiled_cpls(int dtype, int *count);
bool stream_cpl_compiled(int dtype, int cpl);
int default_stream_cpl(int dtype);
int default_stream_wpr(int dtype, int nslots, bool backward);

// one per element type, each in its own translation unit
hipError_t launch_fwd_f32(const FwdArgs &a, const Geometry &g, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs &a, const Geometry &g, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs &a, const Geometry &g, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs &a, const Geometry &g, hipStream_t stream);
hipError_t launch_fwd_f16(const FwdArgs &a, const Geometry &g, hipStream_t stream);
hipError_t launch_bwd_f16(const BwdArgs &a, const Geometry &g, hipStream_t stream);

hipError_t launch_fwd(int dtype, const FwdArgs &a, const Geometry &g, hipStream_t stream);
hipError_t launch_bwd(int dtype, const BwdArgs &a, const Geometry &g, hipStream_t stream);
hipError_t launch_dsink(const DsinkArgs &a, hipStream_t stream);

// Device address of the library's static scratch (JAS_NOALLOC_MAX_ROWS
// floats) on `device`, looked up on the first call for that device.
hipError_t scratch_address(int device, float **out);

}  // namespace jas
