// Fused exact-attention forward for gfx950 (MI355X).
//
// One workgroup of 4 waves owns a tile of 128 queries of one (batch, head);
// each wave owns 32 of them.  K/V tiles of 64 keys stream through LDS
// (double-buffered) past the resident Q fragments, and each tile runs
//   S^T = K Q^T          (bf16 MFMA 32x32x16, fp32 accumulate)
//   mask                 (only on tiles that cross the diagonal or the tail)
//   row max              (in-lane over 32 scores, then one cross-half step)
//   conditional rescale  (only when a row max grows by more than tau = 8)
//   P^T = exp2(S^T c - m_ref), c = scale * log2(e); row sum in fp32
//   O^T += V^T P^T       (P^T used straight from the accumulator registers)
// and the epilogue applies the one final correction O / l and writes
// LSE = (m_ref + log2 l) ln 2.
//
// Passages: tiled online softmax -- zeeklog FlashAttention-4 article, section
// 4 pseudocode; exp2 with the scale folded in, the cubic exp2 share and the
// conditional rescale with one final correction -- hotelren summary, sections
// 3.2-3.3, and danialwang explainer, section 04; computing the transposed
// product so the result is already the next product's operand -- danialwang
// explainer, section 05 (the detail under "一个体现功力的细节").
//
// Why S^T: the 32x32 MFMA accumulator gives lane l the column l % 32.  With
// queries as columns, each lane holds 16 scores of its own query, so the row
// max and sum are in-lane plus one exchange with lane l ^ 32, the per-row
// rescale factor is a per-lane scalar, and the accumulator of S^T is exactly
// the B operand of O^T += V^T P^T (its rows are the contraction index).  The
// A operand V^T needs 8 keys of one d per lane, so V is written to LDS
// transposed, with keys permuted inside each group of 16 so that those 8 keys
// are one 16-byte read.
#include "common.hpp"
#include "kernels.hpp"

namespace fa {
namespace {

constexpr int kFwdBM = 128;   // queries per workgroup
constexpr int kFwdBN = 64;    // keys per K/V tile
constexpr int kFwdWaves = 4;

// Position of local key kl (0..15) inside its 16-key group of a transposed V
// row: bits 2 and 3 swapped, so that accumulator register r of lane half h
// (key 8 (r/4) + 4 h + r % 4) lands at position 8 h + r for r < 8.
__device__ __forceinline__ int vt_pos16(int kl) {
  return (kl & 3) | ((kl >> 3) & 1) << 2 | ((kl >> 2) & 1) << 3;
}
// 16-byte chunk swizzle of a transposed V row (8 chunks of 8 keys): distinct
// chunks for 8 consecutive d (MFMA reads) and for d stepping by 8 (writes).
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

template <int D, bool CAUSAL, int POLYQ>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O,
                                                     float* __restrict__ LSE, FwdParams p) {
  constexpr int BM = kFwdBM, BN = kFwdBN;
  constexpr int KCH = D / 8;            // 16-byte chunks per row
  constexpr int KT_ELEMS = BN * D;      // one K (or V^T) tile, in bf16 elements
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2 * KT_ELEMS];

  // Grid order: consecutive workgroup ids walk heads first, so with B*Hq a
  // multiple of 8 every tile of a head lands on the same XCD (ids are dealt to
  // the 8 XCDs round-robin) and shares K/V in that XCD's L2; query tiles go
  // from last to first so that, under the causal mask, the longest tiles
  // start first.
  const int wg = blockIdx.x;
  const int bh = wg % p.BH;
  const int qb = p.nqb - 1 - wg / p.BH;
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const int hk = hq / p.G;
  const size_t kv_off = ((size_t)b * (p.Hq / p.G) + hk) * (size_t)p.N * D;
  const uint16_t* __restrict__ Qh = Q + (size_t)bh * p.N * D;
  const uint16_t* __restrict__ Kh = K + kv_off;
  const uint16_t* __restrict__ Vh = V + kv_off;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int q0 = qb * BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + n;

  // Q fragments (B operand of S^T = K Q^T): k-step t covers d in [16t, 16t+16),
  // lane half h holds d = 16t + 8h .. +8 of query qi.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qi < p.N) v = *(const u32x4*)(Qh + (size_t)qi * D + 16 * t + 8 * h);
    qf[t] = as_bf16x8(v);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_ref = -__builtin_inff();
  float l_part = 0.f;  // this lane half's share of the row sum

  const int kend = CAUSAL ? min(p.N, q0 + BM) : p.N;
  const int ntiles = (kend + BN - 1) / BN;

  // ---- staging: K row-major, V transposed --------------------------------
  // K: chunk c of row r goes to chunk c ^ (r & 7) (conflict-free MFMA reads
  // of 32 rows at one logical chunk).
  constexpr int K_PER_T = BN * KCH / 256;
  u32x4 kreg[K_PER_T];
  // V: thread owns keys 4g..4g+3 of d-chunk vc (BN/4 * KCH slots).
  constexpr int V_SLOTS = (BN / 4) * KCH;
  const bool v_active = tid < V_SLOTS;
  const int vc = tid % KCH, vg = tid / KCH;
  u32x4 vreg[4];

  auto load_tile = [&](int kt) {
    const int k0 = kt * BN;
#pragma unroll
    for (int s = 0; s < K_PER_T; ++s) {
      const int idx = tid + 256 * s;
      const int r = idx / KCH, c = idx % KCH;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k0 + r < p.N) v = *(const u32x4*)(Kh + (size_t)(k0 + r) * D + c * 8);
      kreg[s] = v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * vg + j;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (v_active && k0 + r < p.N) v = *(const u32x4*)(Vh + (size_t)(k0 + r) * D + vc * 8);
      vreg[j] = v;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = smem[buf];
    uint16_t* vs = smem[buf] + KT_ELEMS;
#pragma unroll
    for (int s = 0; s < K_PER_T; ++s) {
      const int idx = tid + 256 * s;
      const int r = idx / KCH, c = idx % KCH;
      *(u32x4*)(ks + r * D + ((c ^ (r & 7)) * 8)) = kreg[s];
    }
    if (v_active) {
      // 4 keys x 8 d -> 8 rows of V^T, 4 keys (8 bytes) each.
      const int pos = 16 * (vg >> 2) + vt_pos16(4 * (vg & 3));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = vc * 8 + e;
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 out;
        out[0] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
        out[1] = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
        const int chunk = (pos >> 3) ^ vt_swz(d);
        *(u32x2*)(vs + d * BN + chunk * 8 + (pos & 7)) = out;
      }
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) load_tile(kt + 1);
    const int k0 = kt * BN;
    // Tiles wholly above this wave's diagonal contribute nothing.
    const bool skip = CAUSAL && (k0 > qw + 31);
    if (!skip) {
      const uint16_t* ks = smem[buf];
      const uint16_t* vs = smem[buf] + KT_ELEMS;
      // S^T for the two 32-key halves of the tile.
      f32x16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
        const int kr = 32 * sb + n;  // key row this lane feeds (A operand)
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const int c = (2 * t + h) ^ (kr & 7);
          const bf16x8 a = as_bf16x8(*(const u32x4*)(ks + kr * D + c * 8));
          s[sb] = mfma32(a, qf[t], s[sb]);
        }
      }
      // Mask keys past the end and, under causal, keys after the query.
      const bool need_mask = (k0 + BN > p.N) || (CAUSAL && (k0 + BN - 1 > qw));
      if (need_mask) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * sb + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool dead = key >= p.N || (CAUSAL && key > qi);
            if (dead) s[sb][r] = -__builtin_inff();
          }
      }
      // Row max of this tile (both halves end with the full-row value).
      float mx = -__builtin_inff();
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[sb][r], s[sb][r + 1]));
      mx = __builtin_fmaxf(mx, xhalf(mx));
      const float m_new = __builtin_fmaxf(m_ref, mx * p.c);
      // Conditional rescale: taken by the whole wave when any of its rows'
      // max grew by more than tau; each row then moves to its own new max.
      const bool grow = m_new > m_ref + kTau;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = (m_new == -__builtin_inff()) ? 1.f : exp2_hw(m_ref - m_new);
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        m_ref = m_new;
      }
      const float msub = (m_ref == -__builtin_inff()) ? 0.f : m_ref;
      // P^T = exp2(S^T c - m_ref), row sum, and bf16 B operands.
      bf16x8 pb[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = __builtin_fmaf(s[sb][r], p.c, -msub);
          const float e = ((r & 3) < POLYQ) ? exp2_poly(x) : exp2_hw(x);
          s[sb][r] = e;
          l_part += e;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(s[sb][8 * u + 2 * j], s[sb][8 * u + 2 * j + 1]);
          pb[sb][u] = as_bf16x8(w);
        }
      }
      // O^T += V^T P^T.
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = 32 * db + n;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int chunk = (2 * (2 * sb + u) + h) ^ vt_swz(d);
            const bf16x8 a = as_bf16x8(*(const u32x4*)(vs + d * BN + chunk * 8));
            oacc[db] = mfma32(a, pb[sb][u], oacc[db]);
          }
      }
    }
    if (kt + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Final correction: O = O / l, LSE = (m_ref + log2 l) ln 2.
  const float l_tot = l_part + xhalf(l_part);
  if (qi < p.N) {
    const float inv = 1.f / l_tot;
    uint16_t* Oq = O + ((size_t)bh * p.N + qi) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *(u32x2*)(Oq + 32 * db + 8 * g + 4 * h) = w;
      }
    if (h == 0) LSE[(size_t)bh * p.N + qi] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL, int POLYQ>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.BH = a.B * a.Hq;
  p.Hq = a.Hq;
  p.G = a.Hq / a.Hkv;
  p.N = a.N;
  p.nqb = (a.N + kFwdBM - 1) / kFwdBM;
  p.c = a.scale * kLog2e;
  const dim3 grid((unsigned)(p.BH * p.nqb));
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, POLYQ>), grid, dim3(64 * kFwdWaves), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_c(const FwdArgs& a, hipStream_t s) {
  switch (a.poly_quarters) {
    case 0: return launch_fwd_t<D, CAUSAL, 0>(a, s);
    case 1: return launch_fwd_t<D, CAUSAL, 1>(a, s);
    default: return launch_fwd_t<D, CAUSAL, 2>(a, s);
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.D == 64) return a.causal ? launch_fwd_c<64, true>(a, s) : launch_fwd_c<64, false>(a, s);
  return a.causal ? launch_fwd_c<128, true>(a, s) : launch_fwd_c<128, false>(a, s);
}

}  // namespace fa
