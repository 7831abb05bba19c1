// jas_attn.hip -- fixed-order fused attention forward on gfx950 MFMA: the QK
// product, the row softmax of jas_fwd, and the PV product in one kernel.
//
// Method: RL-Kernel PR #453, Summary (the fixed-order softmax sits between
// the QK GEMM and the AV GEMM; P is rounded once, to the tensor dtype) and
// RL-Kernel PR #240, Fixed Reduction Contract (every score and every output
// element has one writer; the head dimension and the keys are accumulated
// in a fixed order, with no split of the key range).
//
// Mapping to CDNA4.  A workgroup of 4 waves owns 64 or 128 queries of one
// (batch, head), each wave one or two blocks of 16 (QB).  Scores are
// computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32 (bf16 or
// fp16): A = 16 keys x 32 dims of K, B = 32 dims x 16 queries of Q (kept in
// registers for the whole row), so lane l holds, for query l%16 of a block,
// four consecutive keys of a 16-key block.  With two query blocks every K
// operand read from LDS (and every V operand in the PV product) feeds two
// MFMAs, which halves the LDS bytes per product, the limit of the one-block
// kernel.  Keys go through the workgroup 32 at a time: K and V (32 keys x
// D each, as they lie in memory) are loaded with coalesced 16-byte loads
// into double-buffered LDS, K two steps and V one step ahead of use, and
// each step issues the next step's QK product before its own softmax work
// (a one-step software pipeline).  LDS row strides are 32 modulo 64 bytes,
// which gfx950 serves without bank conflicts for these reads.  Workgroups
// are renumbered so that one XCD works on neighbouring query blocks of one
// head (its K and V stay in that XCD's L2); with the causal flag a head's
// blocks go longest first.  In
// each 32-key step the A rows are assigned so that lane group g (= l/16)
// holds keys 8g .. 8g + 7 (the first block the first four, the second block
// the next four).  The softmax tile tree is then exact: in-lane pairs and
// quads, the two blocks in-lane, lane groups g and g^1 with
// permlane16_swap, groups {0,1} and {2,3} with permlane32_swap, then the 8
// steps of the 256-key tile in registers -- the balanced pairwise tree over
// the tile's keys in order.  The same registers, rounded to the tensor
// dtype, are the A operand of the PV product (16 queries x 32 keys, lane
// group g holding 8 consecutive keys), so P never leaves the registers; B
// is 32 keys x 16 dims of V, built from the LDS rows of V by gfx950's
// transposed LDS read (ds_read_b64_tr_b16), so V needs no transposed copy.
//
// The softmax is done in two passes over the keys, so that P is exactly the
// row softmax of the binary32 scores (the bits jas_fwd gives on them):
// pass 1 computes each tile's (max, sum), keeps the max in LDS, and merges
// the pair into the query's running state in tile order (then the sink);
// pass 2 recomputes the scores 32 keys at a time, forms P = e * c_t, rounds
// it, and accumulates P V into fp32 registers in key order.  QK is computed
// twice, PV once.  Accumulation inside one MFMA follows the hardware's
// fixed order; every launch computes every output the same way, so results
// do not depend on batch, position or grid.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jas_attn.h"
#include "jas_kernels.h"

namespace jas {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v2i16 __attribute__((ext_vector_type(2)));

constexpr int kAttnWaves = 4;  // waves per workgroup, each on its own queries

template <int DT>
__device__ __forceinline__ f32x4_t mfma32(const u32x4 a, const u32x4 b, const f32x4_t c) {
  if constexpr (DT == 1)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == 1) return pack_bf16(lo, hi);
  else return pack_f16(lo, hi);
}

__device__ __forceinline__ u32x4 bload4(const Buf &b, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(b.r, (int)voff, (int)soff, 0);
}

// Sum over the 64 lanes' groups of 16 (lane groups g = 0..3 in order) as the
// two top levels of a balanced tree: (g0 + g1) + (g2 + g3).
__device__ __forceinline__ float groups4_sum(float v) {
  const f32x2_t p = rows16_pair(v);
  v = p[0] + p[1];
  const f32x2_t h = halves32_pair(v);
  return h[0] + h[1];
}

__device__ __forceinline__ float groups4_max(float v) {
  const f32x2_t p = rows16_pair(v);
  v = fmax2(p[0], p[1]);
  const f32x2_t h = halves32_pair(v);
  return fmax2(h[0], h[1]);
}

// The hardware hands workgroups to the 8 XCDs round-robin (workgroup i to
// XCD i % 8), and each XCD has its own L2.  Renumber so that the workgroups
// on one XCD take consecutive units, i.e. neighbouring query blocks of one
// (batch, head), whose K and V then stay in that XCD's L2.  A bijection on
// [0, G) for any G; which workgroup computes a unit never changes its bytes.
__device__ __forceinline__ int64_t xcd_unit(int64_t bid, int64_t G) {
  const int64_t x = bid % 8, per = G / 8, rem = G % 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + bid / 8;
}

// MASK: an additive mask is given; WRITE: the scores and / or P are written
// out as well (for checking), which the fast path does not carry.  QB: blocks
// of 16 queries per wave.  With QB = 2 each K and V operand read from LDS
// feeds two MFMAs, one per query block, which halves the LDS bytes per
// product.  Every query goes through the same operations, in the same order,
// whatever QB is, so QB never changes a bit of the results.
template <int DT, int D, bool MASK, bool WRITE, int QB>
__global__ __launch_bounds__(kWave * kAttnWaves) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int ESZ = 2;
  constexpr int DS = D / 32;       // k-steps of the QK product
  constexpr int DB = D / 16;       // 16-dim column blocks of the output
  constexpr int SUB = 32;          // keys per staged sub-tile (one PV k-step)
  constexpr int QW = 16 * QB;      // queries per wave
  constexpr int QU = QW * kAttnWaves;  // queries per workgroup
  // LDS rows: a 16-byte read by each lane of 16 rows (lane groups 16 bytes
  // apart) is free of bank conflicts on gfx950 when the row stride is 32
  // modulo 64 bytes (measured; strides 16 modulo 32 bytes cost 4 extra
  // cycles per read): K rows of D + 16 elements.  V rows are D + 16 elements
  // too, which with the row order of vrow() below spreads each transposed
  // read's 8 rows of 32 bytes over different banks
  constexpr int KROW = D + 16;     // LDS row of K (elements)
  constexpr int VROW = D + 16;     // LDS row of V (one key's D dims)
  constexpr int KCH = SUB * D / 8 / (kWave * kAttnWaves);  // 16-byte chunks per thread
  constexpr int VCH = D * SUB / 8 / (kWave * kAttnWaves);
  static_assert(KCH >= 1 && VCH >= 1, "sub-tile smaller than the workgroup");
  __shared__ __align__(16) uint16_t lk[2][SUB * KROW];
  __shared__ __align__(16) uint16_t lv[2][SUB * VROW];
  extern __shared__ float lds_m[];  // per wave T x QW tile maxima (sized at launch)

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane & 15;  // the lane's query in each block (S^T column) and A/B operand row
  const int g = lane >> 4;    // lane group: keys 8g .. 8g+7 of each 32-key step
  const int N = (int)a.N, T = a.T;
  const int Sq = (int)a.Sq;
  const int64_t qgroups = (a.Sq + QU - 1) / QU;  // QU queries per workgroup
  const int64_t units = a.B * a.H * qgroups;
  float *sm = lds_m + w * a.T * QW;
  const bool has_sink = a.sink != nullptr;
  constexpr bool write_all = WRITE;

  for (int64_t u = xcd_unit(blockIdx.x, gridDim.x); u < units; u += gridDim.x) {
    // causal: a head's query blocks in decreasing cost (the last block sees
    // the most keys), so the cheapest units are the last ones dispatched
    const int64_t qg = a.ex.causal ? qgroups - 1 - u % qgroups : u % qgroups, bh = u / qgroups;
    const int64_t h = bh % a.H, b = bh / a.H;
    const int64_t hk = h / (a.H / a.Hkv);
    const int qw = (int)(qg * QU) + QW * w;  // this wave's first query; block qb starts at qw + 16qb
    int qq[QB];                              // this lane's query in each block
    bool qvalid[QB];
    int64_t row[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      qq[qb] = qw + 16 * qb + c16;
      qvalid[qb] = qq[qb] < Sq;
      row[qb] = bh * a.Sq + (qvalid[qb] ? qq[qb] : Sq - 1);
    }

    const Buf kbuf(static_cast<const char *>(a.k) + (b * a.Hkv + hk) * a.N * D * ESZ,
                   (uint32_t)(a.N * D * ESZ));
    const Buf vbuf(static_cast<const char *>(a.v) + (b * a.Hkv + hk) * a.N * D * ESZ,
                   (uint32_t)(a.N * D * ESZ));

    // Q^T operand of block qb (B of the QK product): query qw + 16qb + c16,
    // dims 32ds + 8g .. +7.  The block's buffer ends at the last query, so
    // the lanes of queries past it read 0 through their own offsets.
    u32x4 qv[QB][DS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int q0 = qw + 16 * qb;
      const int nq = Sq - q0 < 0 ? 0 : (Sq - q0 > 16 ? 16 : Sq - q0);
      const Buf qbuf(static_cast<const char *>(a.q) + (bh * a.Sq + q0) * D * ESZ,
                     (uint32_t)(nq * D * ESZ));
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        qv[qb][ds] = bload4(qbuf, (uint32_t)((c16 * D + 8 * g) * ESZ), (uint32_t)(ds * 32 * ESZ));
    }

    // visible keys of the lane's queries, and of the workgroup's last query
    int kend[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      int64_t ke = N;
      if (a.ex.causal) {
        const int64_t off = (int64_t)N - Sq + 1;
        ke = (qq[qb] + off < ke) ? qq[qb] + off : ke;
      }
      if (a.ex.key_len) {
        const int64_t l = a.ex.key_len[b];
        ke = l < ke ? l : ke;
      }
      kend[qb] = (int)(ke < 0 ? 0 : ke);
    }
    int64_t km = N;
    if (a.ex.causal) {
      const int64_t off = (int64_t)N - Sq + 1;
      const int64_t qlast = (qg * QU + QU - 1 < Sq) ? qg * QU + QU - 1 : Sq - 1;
      km = (qlast + off < km) ? qlast + off : km;
    }
    if (a.ex.key_len) {
      const int64_t l = a.ex.key_len[b];
      km = l < km ? l : km;
    }
    int kmax = __builtin_amdgcn_readfirstlane((int)(km < 0 ? 0 : km));
    if (write_all) kmax = N;
    const int tlive = (kmax + kTile - 1) / kTile;  // tiles holding a visible key (same in all waves)
    // keys below the workgroup's smallest cut need no select
    int64_t kn = N;
    if (a.ex.causal) {
      const int64_t off = (int64_t)N - Sq + 1;
      kn = (qg * QU + off < kn) ? qg * QU + off : kn;
    }
    if (a.ex.key_len) {
      const int64_t l = a.ex.key_len[b];
      kn = l < kn ? l : kn;
    }
    const int kmin = __builtin_amdgcn_readfirstlane((int)(kn < 0 ? 0 : kn));
    // the mask of (b, h) as one buffer: the lane's row at q * msq, keys at
    // +key; the buffer ends with the last row's key N - 1, so keys past N of
    // the last row read 0 (they are cut anyway).  With QB > 1 the launch
    // guarantees msq == 0 (one mask row for all queries of the head), so the
    // query blocks share the mask registers.
    Buf mbuf(nullptr, 0u);
    uint32_t moff = 0;
    if constexpr (MASK) {
      mbuf = Buf(a.mask + b * a.msb + h * a.msh, (uint32_t)((((int64_t)Sq - 1) * a.msq + N) * 4));
      moff = (uint32_t)((int64_t)(qvalid[0] ? qq[0] : Sq - 1) * a.msq * 4) + 32u * (uint32_t)g;
    }

    // ---- staging: sub-tile `it` (keys 32*it .. +31) of K, and of V ----
    u32x4 pk[KCH], pv[VCH];
    auto fetch_k = [&](int it) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int ch = tid + c * kWave * kAttnWaves;
        const int r = ch / (D / 8), c8 = ch % (D / 8);
        pk[c] = bload4(kbuf, (uint32_t)((r * D + 8 * c8) * ESZ), (uint32_t)(SUB * it * D * ESZ));
      }
    };
    // key k = 8g + 4hb + r of the sub-tile is kept at LDS row 16hb + 4g + r,
    // so the A rows of one block are 16 consecutive LDS rows
    auto put_k = [&](int buf) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int ch = tid + c * kWave * kAttnWaves;
        const int r = ch / (D / 8), c8 = ch % (D / 8);
        const int pr = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
        *reinterpret_cast<u32x4 *>(&lk[buf][pr * KROW + 8 * c8]) = pk[c];
      }
    };
    // V rows as they are in memory: 16-byte chunks of 8 dims of one key;
    // keys past N read 0 (outside the buffer), so 0 * V adds nothing
    auto fetch_v = [&](int it) {
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const int ch = tid + c * kWave * kAttnWaves;
        const int r = ch / (D / 8), c8 = ch % (D / 8);
        pv[c] = bload4(vbuf, (uint32_t)((r * D + 8 * c8) * ESZ), (uint32_t)(SUB * it * D * ESZ));
      }
    };
    // key r of the sub-tile at LDS row vrow(r): bit 2 flipped for keys with
    // bit 3 set, so that the 8 rows one transposed read touches (keys
    // 8g + 0..3 or 8g + 4..7 of two neighbouring groups g) fall on
    // different banks
    auto vrow = [](int r) { return r ^ (((r >> 3) & 1) << 2); };
    auto put_v = [&](int buf) {
#pragma unroll
      for (int c = 0; c < VCH; ++c) {
        const int ch = tid + c * kWave * kAttnWaves;
        const int r = ch / (D / 8), c8 = ch % (D / 8);
        *reinterpret_cast<u32x4 *>(&lv[buf][vrow(r) * VROW + 8 * c8]) = pv[c];
      }
    };
    // S^T of sub-tile it from LDS buffer buf for every query block: key
    // blocks hb = 0, 1 (keys 32it + 8(c16/4) + 4hb + c16%4 as A rows, LDS
    // rows 16hb + c16), raw dot products.  Each A operand read feeds the
    // MFMAs of all QB query blocks.
    auto qk_sub = [&](int buf, f32x4_t (&s0)[QB], f32x4_t (&s1)[QB]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s0[qb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        s1[qb] = s0[qb];
      }
      // The wave issuing its QK products runs at raised priority, so that
      // the SIMD's other wave fills the matrix core's cycles with its VALU
      // work instead of competing for issue (scheduling only).  Measured on
      // MI355X against the same kernel without it: joint [1,24,4352,128]
      // 0.517 -> 0.507 ms, causal [1,32,8192,128] 1.045 -> 0.996 ms; the
      // same around the PV products made the causal call slower.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const u32x4 k0 = *reinterpret_cast<const u32x4 *>(&lk[buf][c16 * KROW + 32 * ds + 8 * g]);
        const u32x4 k1 = *reinterpret_cast<const u32x4 *>(&lk[buf][(16 + c16) * KROW + 32 * ds + 8 * g]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s0[qb] = mfma32<DT>(k0, qv[qb][ds], s0[qb]);
          s1[qb] = mfma32<DT>(k1, qv[qb][ds], s1[qb]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // the mask of the lane's 8 keys 32it + 8g .. +7: two 16-byte loads, the
    // step's offset in the scalar operand (issued one step ahead of use)
    auto load_mask = [&](int it, u32x4 (&mk)[2]) {
      if constexpr (MASK) {
        mk[0] = bload4(mbuf, moff, (uint32_t)(SUB * 4 * it));
        mk[1] = bload4(mbuf, moff + 16u, (uint32_t)(SUB * 4 * it));
      }
    };
    // scaled, masked and cut scores of the lane's 8 keys 32it + 8g + 4hb + r
    // for query block qb
    auto make_x = [&](int it, int qb, const f32x4_t &s0, const f32x4_t &s1, const u32x4 (&mk)[2],
                      float (&x)[8]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float s = a.scale * ((e < 4) ? s0[e] : s1[e - 4]);
        if constexpr (WRITE) {
          const int key = SUB * it + 8 * g + e;
          if (a.scores && qvalid[qb] && key < N) a.scores[row[qb] * a.N + key] = s;
        }
        x[e] = s;
        if constexpr (MASK) {
          // copy the word out first: a bit cast of a vector element in place
          // reads the vector's first element
          const uint32_t mw = mk[e >> 2][e & 3];
          x[e] = x[e] + __builtin_bit_cast(float, mw);
        }
      }
      if (SUB * it + SUB > kmin) {  // the step reaches some query's cut (uniform)
        const int nv = kend[qb] - (SUB * it + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (e < nv) ? x[e] : kNegInf;
      }
    };

    // ---- pass 1: per tile (max, sum), folded into the row state in tile order ----
    // Software pipeline, one step deep: in step `it` the wave issues the QK
    // product of step it + 1 (K sub-tile it + 1, already in LDS) and the
    // mask of step it + 1, then runs the VALU work of step it on the
    // product issued one step earlier, so the matrix cores and the VALU
    // overlap.  K sub-tile it + 2 is loaded into registers at the start of
    // step it and written to the LDS buffer of sub-tile it (read by every
    // wave in step it - 1) before the step's barrier.
    float M[QB], L[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      M[qb] = kNegInf;
      L[qb] = 0.0f;
    }
    f32x4_t sa[2][QB], sb[2][QB];  // raw S^T of a step (key blocks 0 and 1), by step parity
    u32x4 mk[2][2];
    if (tlive > 0) {
      fetch_k(0);
      put_k(0);
      fetch_k(1);
      put_k(1);
      __syncthreads();
      load_mask(0, mk[0]);
      qk_sub(0, sa[0], sb[0]);
      __syncthreads();  // every wave has read sub-tile 0 before step 0 overwrites it
    }
    for (int t = 0; t < tlive; ++t) {
      float x[QB][8][8];  // [query block][32-key step j][key 8g + e]
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int it = 8 * t + j;
        const int cur = j & 1, nxt = cur ^ 1;  // it is 8t + j: parity of j
        fetch_k(it + 2);
        load_mask(it + 1, mk[nxt]);
        qk_sub(nxt, sa[nxt], sb[nxt]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) make_x(it, qb, sa[cur][qb], sb[cur][qb], mk[cur], x[qb][j]);
        put_k(cur);
        __syncthreads();
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int e = 0; e < 8; e += 2) mx = fmax2(mx, fmax2(x[qb][j][e], x[qb][j][e + 1]));
        const float m = groups4_max(mx);
        const float msafe = (m == kNegInf) ? 0.0f : m;
        float pj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float e8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) e8[e] = exp_(x[qb][j][e] - msafe);
          const float s0 = (e8[0] + e8[1]) + (e8[2] + e8[3]);
          const float s1 = (e8[4] + e8[5]) + (e8[6] + e8[7]);
          pj[j] = groups4_sum(s0 + s1);  // the step's 32 keys
        }
        const float l = ((pj[0] + pj[1]) + (pj[2] + pj[3])) + ((pj[4] + pj[5]) + (pj[6] + pj[7]));
        if (g == 0) sm[t * QW + 16 * qb + c16] = m;
        // merge (m, l) into the row state
        const float Mn = fmax2(M[qb], m);
        if (Mn == kNegInf) {
          M[qb] = kNegInf;
          L[qb] = 0.0f;
        } else {
          const float fa = (M[qb] == kNegInf) ? 0.0f : exp_(M[qb] - Mn);
          const float fb = (m == kNegInf) ? 0.0f : exp_(m - Mn);
          const float La = L[qb] * fa;
          const float lb = l * fb;
          L[qb] = La + lb;
          M[qb] = Mn;
        }
      }
    }
    // tiles past every visible key of the workgroup hold only -inf: (-inf, 0)
    // states, which leave (M, L) as they are
    const float sigma = has_sink ? a.sink[h] : 0.0f;
    float invL[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (has_sink) {
        const float Mn = fmax2(M[qb], sigma);
        if (Mn == kNegInf) {
          M[qb] = kNegInf;
          L[qb] = 0.0f;
        } else {
          const float fa = (M[qb] == kNegInf) ? 0.0f : exp_(M[qb] - Mn);
          const float fb = (sigma == kNegInf) ? 0.0f : exp_(sigma - Mn);
          const float La = L[qb] * fa;
          const float lb = 1.0f * fb;
          L[qb] = La + lb;
          M[qb] = Mn;
        }
      }
      invL[qb] = (L[qb] == 0.0f) ? 0.0f : 1.0f / L[qb];
      if (g == 0 && qvalid[qb]) {
        if (has_sink) a.p_sink[row[qb]] = (sigma == kNegInf) ? 0.0f : exp_(sigma - M[qb]) * invL[qb];
        if (a.lse) a.lse[row[qb]] = (L[qb] == 0.0f) ? kNegInf : M[qb] + ln_(L[qb]);
      }
    }

    // ---- pass 2: P = e * c_t rounded to the dtype, O += P V, sub-tile by sub-tile ----
    f32x4_t o[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // the same pipeline: step it issues QK of step it + 1, forms P of step
    // it, accumulates P V of step it (V sub-tile it in LDS), and writes K
    // sub-tile it + 2 and V sub-tile it + 1 to LDS before its barrier
    if (tlive > 0) {
      fetch_k(0);
      put_k(0);
      fetch_k(1);
      put_k(1);
      fetch_v(0);
      put_v(0);
      __syncthreads();
      load_mask(0, mk[0]);
      qk_sub(0, sa[0], sb[0]);
      __syncthreads();
    }
    for (int t = 0; t < tlive; ++t) {
      float msafe[QB], ct[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mt = sm[t * QW + 16 * qb + c16];
        msafe[qb] = (mt == kNegInf) ? 0.0f : mt;
        ct[qb] = (mt == kNegInf) ? 0.0f : exp_(mt - M[qb]) * invL[qb];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int it = 8 * t + j;
        const int cur = j & 1, nxt = cur ^ 1;
        fetch_k(it + 2);
        fetch_v(it + 1);
        load_mask(it + 1, mk[nxt]);
        qk_sub(nxt, sa[nxt], sb[nxt]);
        u32x4 pa[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float x[8], p[8];
          make_x(it, qb, sa[cur][qb], sb[cur][qb], mk[cur], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = exp_(x[e] - msafe[qb]) * ct[qb];
          pa[qb] = u32x4{pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3]), pack2<DT>(p[4], p[5]),
                         pack2<DT>(p[6], p[7])};
          if constexpr (WRITE) {
            if (a.probs && qvalid[qb]) {
              uint16_t *prow = static_cast<uint16_t *>(a.probs) + row[qb] * a.N;
              const int key0 = SUB * it + 8 * g;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (key0 + e < N) prow[key0 + e] = (uint16_t)(pa[qb][e >> 1] >> (16 * (e & 1)));
            }
          }
        }
        // B operand: keys 32it + 8g .. +7 of dims 16db + c16, shared by the
        // query blocks, built by two transposed LDS reads (gfx950
        // ds_read_b64_tr_b16).  In each group of 16 lanes, lane j names the
        // 4 dims 16db + 4(j%4) .. +3 of key 8g + j/4 (then 8g + 4 + j/4);
        // the read hands lane i the 4 values of dim 16db + i for those 4
        // keys, in key order.
        const int vk0 = vrow(8 * g + (c16 >> 2)), vk1 = vrow(8 * g + 4 + (c16 >> 2));
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int dc = 16 * db + 4 * (c16 & 3);
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16 *)(&lv[cur][vk0 * VROW + dc]));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16 *)(&lv[cur][vk1 * VROW + dc]));
          const u32x4 vv = {__builtin_bit_cast(uint32_t, v2i16{lo[0], lo[1]}),
                            __builtin_bit_cast(uint32_t, v2i16{lo[2], lo[3]}),
                            __builtin_bit_cast(uint32_t, v2i16{hi[0], hi[1]}),
                            __builtin_bit_cast(uint32_t, v2i16{hi[2], hi[3]})};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32<DT>(pa[qb], vv, o[qb][db]);
        }
        put_k(cur);
        put_v(nxt);
        __syncthreads();
      }
    }

    // ---- O rows qw + 16qb + 4g + r, dims 16db + c16: round once, write ----
    uint16_t *orow = static_cast<uint16_t *>(a.out) + bh * a.Sq * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int oq = qw + 16 * qb + 4 * g + r;
        if (oq < Sq) {
#pragma unroll
          for (int db = 0; db < DB; db += 2) {
            const uint32_t w2 = pack2<DT>(o[qb][db][r], o[qb][db + 1][r]);
            orow[(int64_t)oq * D + 16 * db + c16] = (uint16_t)(w2 & 0xffffu);
            orow[(int64_t)oq * D + 16 * (db + 1) + c16] = (uint16_t)(w2 >> 16);
          }
        }
      }
    }
    __syncthreads();  // LDS is reused by the workgroup's next unit
  }
}

// Query blocks per wave.  Two blocks halve the LDS operand bytes per
// product but need 210-255 registers per lane (two waves per SIMD instead
// of three or four) and twice the tile-maximum LDS.  The default takes them
// for the fast path when the workgroup's LDS stays within 64 KB and there
// are units enough for one round of the chip's workgroup slots (256 CUs x
// 2).  Measured on MI355X, joint shape [1,24,4352,128] with its padding
// mask: 0.584 ms with one block, 0.514 ms with two; causal
// [1,32,8192,128] with the sink: 1.27 ms and 1.03 ms; head dimension 64,
// the same two shapes: 0.429 / 0.377 ms and 0.815 / 0.700 ms.  The query
// blocks share one set of mask registers, so a mask that varies by query
// always runs with one block, whatever was asked.  Every choice gives the
// same bits.
template <int D>
int attn_query_blocks(const AttnArgs &a, bool write, int asked) {
  constexpr size_t kStatic = 2 * (2 * 32 * (D + 16) * 2);  // lk + lv bytes
  if (a.mask != nullptr && a.msq != 0) return 1;
  if (kStatic + (size_t)kAttnWaves * a.T * 32 * sizeof(float) > 65536) return 1;
  if (asked != 0) return asked;
  if (write) return 1;
  const int64_t units2 = a.B * a.H * ((a.Sq + 127) / 128);
  if (units2 < 2 * 256) return 1;
  return 2;
}

template <int DT, int D, int QB>
hipError_t attn_launch_qb(const AttnArgs &a, hipStream_t st) {
  int64_t blocks = a.B * a.H * ((a.Sq + 64 * QB - 1) / (64 * QB));
  if (blocks > 0x7fffffff) blocks = 0x7fffffff;
  const dim3 grid((unsigned)blocks), block(kWave * kAttnWaves);
  const size_t dyn = (size_t)kAttnWaves * a.T * 16 * QB * sizeof(float);
  const bool mask = a.mask != nullptr, write = a.probs != nullptr || a.scores != nullptr;
  if (mask) {
    if (write) hipLaunchKernelGGL((attn_fwd_kernel<DT, D, true, true, QB>), grid, block, dyn, st, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<DT, D, true, false, QB>), grid, block, dyn, st, a);
  } else {
    if (write) hipLaunchKernelGGL((attn_fwd_kernel<DT, D, false, true, QB>), grid, block, dyn, st, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<DT, D, false, false, QB>), grid, block, dyn, st, a);
  }
  return hipGetLastError();
}

template <int DT, int D>
hipError_t attn_launch(const AttnArgs &a, int qblocks, hipStream_t st) {
  const bool write = a.probs != nullptr || a.scores != nullptr;
  qblocks = attn_query_blocks<D>(a, write, qblocks);
  if (qblocks == 2) return attn_launch_qb<DT, D, 2>(a, st);
  return attn_launch_qb<DT, D, 1>(a, st);
}

}  // namespace

hipError_t launch_attn_fwd(int dtype, const AttnArgs &a, int qblocks, hipStream_t st) {
  if (dtype == 1) return a.D == 64 ? attn_launch<1, 64>(a, qblocks, st) : attn_launch<1, 128>(a, qblocks, st);
  return a.D == 64 ? attn_launch<2, 64>(a, qblocks, st) : attn_launch<2, 128>(a, qblocks, st);
}

}  // namespace jas
