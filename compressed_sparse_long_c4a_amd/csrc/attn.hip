// Sparse multi-query attention with K = V over top-k compressed entries plus the sliding
// window, followed by inverse RoPE at the query position.
//
// [vLLM-V4] section 2: keys and values are the same vectors (2x saving); queries attend to
// the top-k compressed tokens plus 128 uncompressed window tokens.  [vLLM-V4] appendix, why
// inverse RoPE: with v_n = k_n = R_n k the output must be multiplied by R_m^{-1}, leaving
// R_{n-m}.  [vLLM-V4] appendix, exact k values: c128a attends to every entry (top-k = 8192).
//
// Kernel 1 (attn_partial), grid (row split, 16-head group, query), 4 waves = 2 pairs:
//   the addresses (and fp8 scales) of the split's rows are resolved once into LDS; each pair
//   of waves walks its own 32-row blocks (blocks p, p+2, ...) with a private online softmax,
//   and the two waves of a pair split the row dimensions in halves: each computes the partial
//   logits over its half, the halves are summed through LDS (one barrier per block, double
//   buffered), and each wave accumulates the output for its half of the dims.  The two pairs
//   are merged through LDS at the end; one partial (m, l, O) per head leaves the workgroup.
//   Per 32-row block (two 16-row tiles T0, T1):
//     QK : S^T[16 rows x 16 heads] = R_T . Q^T on MFMA 16x16x32 bf16.  Lane (r, g) holds row
//          r of the tile, 8 dims per k-step, loaded straight from HBM: the row gather and the
//          MFMA operand layout coincide.
//     PV : O^T[dims x heads] += R^T . P^T.  The transposed operand R^T is produced on the
//          matrix cores by a "selection" MFMA, R_T . Sel_h with Sel_h a 0/1 matrix picking 16
//          of the 32 dims of a k-step: its output layout (4 rows x 1 dim per lane) is exactly
//          the A layout PV needs, with rows of T0 in slots 0-3 and rows of T1 in slots 4-7.
//          P^T comes straight from the QK output registers in the same row order.  P is split
//          into bf16 hi + lo parts (two MFMAs) so PV keeps ~16 significant bits.
//   fp8 rows (code * per-row scale): codes widen exactly to bf16; the scale multiplies the
//   logit and P.  float32 rows / queries are split hi + lo as well.
// Kernel 2 (attn_merge), grid (4-head group, query), one wave per head: combines the splits
//   by their softmax statistics, normalises, applies R_t^{-1} to the last rope_dims dims
//   (angles formed and reduced in float64) and writes out / lse.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplits = 256;
constexpr int kRowsPerSplit = 1024;  // most rows a workgroup handles (addresses staged in LDS)

struct Args {
  int batch, n_heads, ratio, k, has_topk, window, n_max, rows_per_split, splits, hgp;
  const int32_t* cu_q;
  const int32_t* q_pos;
  const void* q;
  const int32_t* topk;
  DevCache kv, swa;
  float sm_scale2;  // softmax_scale * log2(e)
  float* part_o;    // [total_q][splits][hgp][DIM]
  float* part_ml;   // [total_q][splits][hgp][2]  (m in log2 units, l)
};

__device__ __forceinline__ bf16x8 f32x8_to_bf16(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}


// Half a row (HKS k-steps of 32 dims) of one 16-row tile as seen by lane (r, g): the 8 dims
// 32 ks + 8 g .. +7 of row r for each of its k-steps.
template <int DT, int HKS>
struct HalfTile {
  static constexpr int NREG = DT == CSA_FP8_E4M3 ? HKS : (DT == CSA_BF16 ? HKS : 1);
  typedef typename std::conditional<DT == CSA_FP8_E4M3, uint2, uint4>::type Word;
  Word d[NREG];
  const float* f32row;  // float32 rows are re-read per k-step instead of held in registers

  // `row` is always a loadable row (padding rows point at a safe row and are masked later).
  __device__ __forceinline__ void load(const char* row, int ks0, int g) {
    if constexpr (DT == CSA_F32) {
      f32row = (const float*)row + 32 * ks0 + 8 * g;
    } else {
      constexpr int ESZ = DT == CSA_BF16 ? 2 : 1;
      const char* base = row + (32 * ks0 + 8 * g) * ESZ;
#pragma unroll
      for (int kk = 0; kk < HKS; ++kk) d[kk] = *(const Word*)(base + 32 * kk * ESZ);
    }
  }

  // bf16 operand for local k-step kk (exact for bf16 and fp8 rows); lo = residual of float32 rows.
  __device__ __forceinline__ void frag(int kk, bf16x8& hi, bf16x8& lo) const {
    if constexpr (DT == CSA_BF16) {
      hi = __builtin_bit_cast(bf16x8, d[kk]);
    } else if constexpr (DT == CSA_FP8_E4M3) {
      hi = fp8x8_to_bf16x8(d[kk].x, d[kk].y);
    } else {
      float x[8];
      {
        const float4 a = *(const float4*)(f32row + 32 * kk);
        const float4 b = *(const float4*)(f32row + 32 * kk + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      }
      hi = f32x8_to_bf16(x);
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = x[i] - (float)hi[i];
      lo = f32x8_to_bf16(r);
    }
  }
};

template <int DT, int QDT, int DIM>
__global__ __launch_bounds__(256) void attn_partial(Args a) {
  constexpr int NKS = DIM / 32;
  constexpr int HKS = NKS / 2;  // k-steps per wave of a pair
  constexpr bool ROW_LO = DT == CSA_F32;
  constexpr bool Q_LO = QDT == CSA_F32;
  // byte offset of each row from the main cache's row base (window rows included), so every
  // row address is derived from a kernel argument and the loads are known to be global
  __shared__ int64_t off_sh[kRowsPerSplit];
  __shared__ float scale_sh[kRowsPerSplit];  // row scale (1 for bf16/f32 rows); 0 marks padding
  __shared__ float xs[2][4][64][8];  // partial logits, [buffer][wave][lane][T*4 + jj]
  // bf16 / fp8 rows: each wave's bf16 half-rows of the current block (row stride padded by 16 B),
  // read back transposed for PV; the merge at the end reuses the space.  float32 rows use the
  // selection MFMA instead and need only the merge buffer.
  constexpr int TROW = (DIM / 2) * 2 + 16;          // bytes per half-row in LDS
  constexpr int TILE_BYTES = ROW_LO ? 0 : 4 * 32 * TROW;
  constexpr int MERGE_BYTES = 16 * (DIM + 4) * 4;
  __shared__ __attribute__((aligned(16))) char tile_sh[TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES];
  float (*o_sh)[DIM + 4] = reinterpret_cast<float (*)[DIM + 4]>(tile_sh);
  __shared__ float ml_sh[2][16][2];

  const int s = blockIdx.x, hg = blockIdx.y, qi = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int pair = wv >> 1, half = wv & 1;
  const int ln = lane & 15, lg = lane >> 4;
  const int b = seq_of_wave(a.cu_q, a.batch, qi);
  const int t = a.q_pos[qi];
  const int n_vis = min((t + 1) / a.ratio, a.n_max);
  const int n_c = a.has_topk ? a.k : n_vis;
  const int n_w = min(a.window, t + 1);
  const int n_rows = n_c + n_w;
  const int r_begin = s * a.rows_per_split;
  // a query without any visible row (no window and no entry yet) attends to nothing
  const int nrows = (n_w > 0 || n_vis > 0) ? max(0, min(a.rows_per_split, n_rows - r_begin)) : 0;
  const int H = a.n_heads;
  const int ks0 = half * HKS;
  constexpr int ESZ = DT == CSA_F32 ? 4 : (DT == CSA_BF16 ? 2 : 1);

  // Q^T as the B operand: lane (head ln, group lg) holds q[h][32 ks + 8 lg + 0..7].
  bf16x8 qb[HKS], qb_lo[Q_LO ? HKS : 1];
  {
    const int h = 16 * hg + ln;
#pragma unroll
    for (int kk = 0; kk < HKS; ++kk) {
      const int d0 = 32 * (ks0 + kk) + 8 * lg;
      if constexpr (QDT == CSA_BF16) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (h < H) v = *(const uint4*)((const uint16_t*)a.q + ((int64_t)qi * H + h) * DIM + d0);
        qb[kk] = __builtin_bit_cast(bf16x8, v);
      } else {
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (h < H) {
          const float* src = (const float*)a.q + ((int64_t)qi * H + h) * DIM + d0;
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = src[i];
        }
        qb[kk] = f32x8_to_bf16(x);
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = x[i] - (float)qb[kk][i];
        if constexpr (Q_LO) qb_lo[kk] = f32x8_to_bf16(r);
      }
    }
  }
  // ---- resolve the split's rows once: address and scale, padding rows -> a safe row.
  // Each thread owns up to kRowsPerSplit / 256 rows; the list reads, then the block-table
  // reads, then the scale reads of all its rows are issued together.
  if (nrows > 0) {  // (all staged positions are then rows of this query)
    constexpr int RPT = kRowsPerSplit / 256;
    const int64_t swa_off = (int64_t)((uintptr_t)a.swa.rows - (uintptr_t)a.kv.rows);
    const int64_t safe = n_w > 0 ? swa_off + phys_row(a.swa, b, t) * (DIM * ESZ)
                                 : phys_row(a.kv, b, max(n_vis - 1, 0)) * (DIM * ESZ);
    int ent[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = tid + 256 * u;
      const int pos = r_begin + min(i, nrows - 1);
      ent[u] = pos < n_c ? (a.has_topk ? a.topk[(int64_t)qi * a.k + pos] : pos) : -1;
    }
    int64_t prow[RPT];
    bool is_kv[RPT], ok[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = tid + 256 * u;
      const int pos = r_begin + min(i, nrows - 1);
      is_kv[u] = pos < n_c;
      ok[u] = i < nrows && (!is_kv[u] || (ent[u] >= 0 && ent[u] < n_vis));
      prow[u] = is_kv[u] ? (ok[u] ? phys_row(a.kv, b, ent[u]) : 0)
                         : phys_row(a.swa, b, t - n_w + 1 + (pos - n_c));
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = tid + 256 * u;
      if (i < nrows) {
        const int64_t base = is_kv[u] ? 0 : swa_off;
        float sc = 0.f;
        if (ok[u]) {
          if constexpr (DT == CSA_FP8_E4M3) sc = (is_kv[u] ? a.kv.scales : a.swa.scales)[prow[u]];
          else sc = 1.0f;
        }
        off_sh[i] = ok[u] ? base + prow[u] * (DIM * ESZ) : safe;
        scale_sh[i] = sc;
      }
    }
  }

  // Sel_h as the B operand (float32 rows only): slot (lg, j) -> output column 8 (lg - 2h) + j
  // for lg in {2h, 2h+1}.
  bf16x8 sel[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sel[hh][j] = (__bf16)((lg == 2 * hh + (ln >> 3) && j == (ln & 7)) ? 1.0f : 0.0f);
  }

  f32x4 o[HKS][2];
#pragma unroll
  for (int kk = 0; kk < HKS; ++kk) {
    o[kk][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    o[kk][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();

  const int nblocks = (nrows + 31) >> 5;
  const int iters = (nblocks + 1) >> 1;
  // Row loads are unconditional (clamped to the split's last row, which is always loadable):
  // the wait counters then keep the next block in flight while this one is computed.
  auto load_block = [&](int it, HalfTile<DT, HKS>* tl) {
    const int bi = 2 * min(it, iters - 1) + pair;
#pragma unroll
    for (int T = 0; T < 2; ++T)
      tl[T].load((const char*)a.kv.rows + off_sh[min(32 * bi + 16 * T + ln, nrows - 1)], ks0, lg);
  };

  auto process_block = [&](int it, const HalfTile<DT, HKS>* tile, int buf) {
    const int bi = 2 * it + pair;
    const bool active = bi < nblocks;
    const int row0 = 32 * bi;
    // partial S^T = R_half . Q_half^T
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < HKS; ++kk) {
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        bf16x8 rh, rl;
        tile[T].frag(kk, rh, rl);
        if constexpr (!ROW_LO)
          *(bf16x8*)(tile_sh + wv * 32 * TROW + (16 * T + ln) * TROW + 2 * (32 * kk + 8 * lg)) = rh;
        sacc[T] = mfma16x16x32(rh, qb[kk], sacc[T]);
        if constexpr (Q_LO) sacc[T] = mfma16x16x32(rh, qb_lo[kk], sacc[T]);
        if constexpr (ROW_LO) sacc[T] = mfma16x16x32(rl, qb[kk], sacc[T]);
      }
    }
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) xs[buf][wv][lane][4 * T + jj] = sacc[T][jj];
    barrier_lds();  // the next block's row loads stay in flight
    float z[2][4], sc[2][4];
    float mloc = -INFINITY;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float sum = xs[buf][2 * pair][lane][4 * T + jj] + xs[buf][2 * pair + 1][lane][4 * T + jj];
        const int r = row0 + 16 * T + 4 * lg + jj;
        const float rs = (active && r < nrows) ? scale_sh[r] : 0.f;
        sc[T][jj] = rs;
        z[T][jj] = rs != 0.f ? sum * rs * a.sm_scale2 : -INFINITY;
        mloc = fmaxf(mloc, z[T][jj]);
      }
    }
    if (!active) return;
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float m_new = fmaxf(m_run, mloc);
    if (m_new == -INFINITY) return;  // every row so far is padding (uniform per wave)
    // v_exp_f32 directly: arguments are <= 0, and 2^-inf = 0 covers an empty running max and
    // padding rows
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float pv[8];
    float psum = 0.f;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float p = __builtin_amdgcn_exp2f(z[T][jj] - m_new);
        psum += p;
        pv[4 * T + jj] = p * sc[T][jj];
      }
    }
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.0f)) {  // rescale only when some head's running max moved
#pragma unroll
      for (int kk = 0; kk < HKS; ++kk) {
        o[kk][0] *= alpha;
        o[kk][1] *= alpha;
      }
    }
    bf16x8 p_hi = f32x8_to_bf16(pv), p_lo;
    {
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = pv[i] - (float)p_hi[i];
      p_lo = f32x8_to_bf16(r);
    }
    if constexpr (!ROW_LO) {
      // O^T += R^T . P^T over this wave's half of the dims.  The A operand (16 dims x 8 rows per
      // lane) is read transposed from the wave's LDS tile: two ds_read_b64_tr_b16 per fragment,
      // the first over rows 4 lg .. 4 lg + 3 of T0 and the second over the same rows of T1,
      // which is the row order of P^T in the softmax registers.
      __attribute__((address_space(3))) char* tbase =
          (__attribute__((address_space(3))) char*)(tile_sh + wv * 32 * TROW);
      typedef short s16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int kk = 0; kk < HKS; ++kk) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int col = 2 * (32 * kk + 16 * hh + 4 * (ln & 3));
          const int r0 = 4 * lg + (ln >> 2);
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(tbase + r0 * TROW + col));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(tbase + (16 + r0) * TROW + col));
          const bf16x8 at = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[kk][hh] = mfma16x16x32(at, p_hi, o[kk][hh]);
          o[kk][hh] = mfma16x16x32(at, p_lo, o[kk][hh]);
        }
      }
    } else {
      // float32 rows: R^T made by the selection MFMA from the register tiles (hi and lo parts)
#pragma unroll
      for (int kk = 0; kk < HKS; ++kk) {
        bf16x8 r0h, r0l, r1h, r1l;
        tile[0].frag(kk, r0h, r0l);
        tile[1].frag(kk, r1h, r1l);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          const f32x4 c0 = mfma16x16x32(r0h, sel[hh], zero);
          const f32x4 c1 = mfma16x16x32(r1h, sel[hh], zero);
          const f32x4 d0 = mfma16x16x32(r0l, sel[hh], zero);
          const f32x4 d1 = mfma16x16x32(r1l, sel[hh], zero);
          bf16x8 at, al;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            at[jj] = (__bf16)c0[jj];
            at[4 + jj] = (__bf16)c1[jj];
            al[jj] = (__bf16)d0[jj];
            al[4 + jj] = (__bf16)d1[jj];
          }
          o[kk][hh] = mfma16x16x32(at, p_hi, o[kk][hh]);
          o[kk][hh] = mfma16x16x32(at, p_lo, o[kk][hh]);
          o[kk][hh] = mfma16x16x32(al, p_hi, o[kk][hh]);
        }
      }
    }
  };

  if (iters > 0) {
    HalfTile<DT, HKS> ta[2], tb[2];
    load_block(0, ta);
    for (int it = 0; it < iters; it += 2) {
      load_block(it + 1, tb);
      process_block(it, ta, 0);
      load_block(it + 2, ta);
      if (it + 1 < iters) process_block(it + 1, tb, 1);
    }
  }

  // ---- merge the two pairs through LDS (the two waves of a pair hold identical m and l)
  __syncthreads();  // the merge buffer reuses the row tiles
  float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (half == 0 && lg == 0) {
    ml_sh[pair][ln][0] = m_run;
    ml_sh[pair][ln][1] = l_tot;
  }
  __syncthreads();
  const float M = fmaxf(ml_sh[0][ln][0], ml_sh[1][ln][0]);
  const float f = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);
  for (int p = 1; p >= 0; --p) {
    if (pair == p) {
#pragma unroll
      for (int kk = 0; kk < HKS; ++kk) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            // output column m of the selection is dim 32 ks + 16 hh + m
            const int d = 32 * (ks0 + kk) + 16 * hh + 4 * lg + jj;
            const float v = f * o[kk][hh][jj];
            if (p == 1) o_sh[ln][d] = v; else o_sh[ln][d] += v;
          }
        }
      }
    }
    __syncthreads();
  }
  const int64_t pbase = ((int64_t)qi * a.splits + s) * a.hgp + 16 * hg;
  for (int i = tid; i < 16 * DIM / 4; i += 256) {
    const int h = i / (DIM / 4), d = 4 * (i - h * (DIM / 4));
    *(float4*)(a.part_o + (pbase + h) * DIM + d) =
        make_float4(o_sh[h][d], o_sh[h][d + 1], o_sh[h][d + 2], o_sh[h][d + 3]);
  }
  if (tid < 16) {
    const int h = tid;
    const float m0 = ml_sh[0][h][0], m1 = ml_sh[1][h][0];
    const float Mh = fmaxf(m0, m1);
    float L = 0.f;
    if (m0 != -INFINITY) L += exp2f(m0 - Mh) * ml_sh[0][h][1];
    if (m1 != -INFINITY) L += exp2f(m1 - Mh) * ml_sh[1][h][1];
    a.part_ml[(pbase + h) * 2 + 0] = Mh;
    a.part_ml[(pbase + h) * 2 + 1] = L;
  }
}

struct MergeArgs {
  int n_heads, splits, hgp, dim, rope_dims;
  const int32_t* q_pos;
  const float* part_o;
  const float* part_ml;
  float* out;
  float* lse;
  RopeTable rope;
};

// One wave per (query, head): split weights from the partial statistics, weighted sum of the
// partial outputs, normalisation and R_t^{-1} on the last rope_dims dims.  Each lane owns the
// float4 columns lane, lane + 64, lane + 128 of the row; the partial rows of a round of splits
// are loaded before the statistics are read, so both memory trips overlap.  No LDS, no
// workgroup barrier.
constexpr int kMergeCols = 3;   // float4 columns per lane: rows of up to 768 dims
constexpr int kMergeRound = 8;  // splits whose partial rows are loaded together

__global__ __launch_bounds__(256) void attn_merge(MergeArgs a) {
  const int qi = blockIdx.y, lane = threadIdx.x & 63;
  const int h = 4 * blockIdx.x + (threadIdx.x >> 6);
  if (h >= a.n_heads) return;  // whole waves
  const int dim4 = a.dim / 4;
  const int64_t stride4 = (int64_t)a.hgp * dim4;  // float4s between splits of one head
  const int64_t qbase = (int64_t)qi * a.splits;
  const float4* src = (const float4*)a.part_o + (qbase * a.hgp + h) * dim4;
  const float* ml = a.part_ml + (qbase * a.hgp + h) * 2;  // split s at ml[s * hgp * 2]
  const int64_t mls = (int64_t)a.hgp * 2;
  int col[kMergeCols];
#pragma unroll
  for (int j = 0; j < kMergeCols; ++j) col[j] = min(lane + 64 * j, dim4 - 1);
  float4 v[kMergeRound][kMergeCols];
  auto load_round = [&](int s0) {  // clamped, unconditional: every load of the round in flight
#pragma unroll
    for (int u = 0; u < kMergeRound; ++u) {
      const int64_t sb = (int64_t)min(s0 + u, a.splits - 1) * stride4;
#pragma unroll
      for (int j = 0; j < kMergeCols; ++j) v[u][j] = src[sb + col[j]];
    }
  };
  load_round(0);
  const int t = a.q_pos[qi];

  // M = max_s m_s (log2 units), L = sum_s 2^(m_s - M) l_s
  float M = -INFINITY;
  for (int s = lane; s < a.splits; s += 64) M = fmaxf(M, ml[s * mls]);
  M = wave_max(M);
  float L = 0.f;
  for (int s = lane; s < a.splits; s += 64) {
    const float m = ml[s * mls];
    L += (m == -INFINITY) ? 0.f : exp2f(m - M) * ml[s * mls + 1];
  }
  L = wave_sum(L);
  if (a.lse && lane == 0) a.lse[(int64_t)qi * a.n_heads + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;

  float4 acc[kMergeCols];
#pragma unroll
  for (int j = 0; j < kMergeCols; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  float wl = 0.f;  // weight of split 64 g + lane for the current group g
  for (int s0 = 0; s0 < a.splits; s0 += kMergeRound) {
    if (s0 > 0) load_round(s0);
    if ((s0 & 63) == 0) {
      const int s = s0 + lane;
      const float m = s < a.splits ? ml[s * mls] : -INFINITY;
      wl = (m == -INFINITY) ? 0.f : exp2f(m - M);
    }
#pragma unroll
    for (int u = 0; u < kMergeRound; ++u) {
      const float w = s0 + u < a.splits
          ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), (s0 & 63) + u))
          : 0.f;
#pragma unroll
      for (int j = 0; j < kMergeCols; ++j) {
        acc[j].x = fmaf(w, v[u][j].x, acc[j].x);
        acc[j].y = fmaf(w, v[u][j].y, acc[j].y);
        acc[j].z = fmaf(w, v[u][j].z, acc[j].z);
        acc[j].w = fmaf(w, v[u][j].w, acc[j].w);
      }
    }
  }

  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const int rope0 = a.dim - a.rope_dims;  // first rotated dim
  float* orow = a.out + ((int64_t)qi * a.n_heads + h) * a.dim;
#pragma unroll
  for (int j = 0; j < kMergeCols; ++j) {
    if (lane + 64 * j >= dim4) continue;
    const int d = 4 * (lane + 64 * j);
    float4 r = make_float4(acc[j].x * inv, acc[j].y * inv, acc[j].z * inv, acc[j].w * inv);
    if (d >= rope0) {  // pairs (d, d+1) and (d+2, d+3) by -t theta_i
      float c0, s0, c1, s1;
      rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2], c0, s0);
      rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2 + 1], c1, s1);
      r = make_float4(r.x * c0 - r.y * s0, r.x * s0 + r.y * c0, r.z * c1 - r.w * s1, r.z * s1 + r.w * c1);
    }
    *(float4*)(orow + d) = r;
  }
}

template <int DT, int QDT, int DIM>
void launch_partial(const Args& args, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_partial<DT, QDT, DIM>), grid, dim3(256), 0, stream, args);
}

template <int DT, int QDT>
void launch_dim(const Args& args, int dim, dim3 grid, hipStream_t stream) {
  if (dim == 576) launch_partial<DT, QDT, 576>(args, grid, stream);
  else launch_partial<DT, QDT, 512>(args, grid, stream);
}

template <int DT>
void launch_q(const Args& args, int qdt, int dim, dim3 grid, hipStream_t stream) {
  if (qdt == CSA_BF16) launch_dim<DT, CSA_BF16>(args, dim, grid, stream);
  else launch_dim<DT, CSA_F32>(args, dim, grid, stream);
}

}  // namespace

AttnPlan attn_plan(int total_q, int n_heads, int ratio, int has_topk, int k, int max_context,
                   int window) {
  AttnPlan p{};
  const int64_t n_max = max_context / ratio;
  p.max_rows = (has_topk ? (int64_t)k : n_max) + std::min<int64_t>(window, max_context);
  p.head_groups = (n_heads + 15) / 16;
  const int64_t blocks32 = std::max<int64_t>(1, (p.max_rows + 31) / 32);
  const int64_t units = (int64_t)total_q * p.head_groups;
  // aim at one 256-thread workgroup per compute unit (256 CUs), at least 4 blocks per group
  int64_t bpw = std::max<int64_t>(4, (blocks32 * units + 255) / 256);
  bpw = std::min<int64_t>(std::min(bpw, blocks32), kRowsPerSplit / 32);
  // callers keep max_rows <= kMaxSplits * kRowsPerSplit, so splits <= kMaxSplits
  const int64_t splits = (blocks32 + bpw - 1) / bpw;
  p.splits = (int)splits;
  p.rows_per_split = (int)(bpw * 32);
  return p;
}

size_t attn_workspace_bytes(int total_q, int n_heads, int dim, const AttnPlan& p) {
  (void)n_heads;
  const size_t slots = (size_t)total_q * p.splits * p.head_groups * 16;
  const size_t ob = (slots * dim * sizeof(float) + 255) & ~(size_t)255;
  return ob + slots * 2 * sizeof(float);
}

hipError_t launch_sparse_attn(const AttnLaunch& L, const AttnPlan& p, void* workspace,
                              hipStream_t stream) {
  const int dim = L.kv->dim;
  Args a{};
  a.batch = L.batch;
  a.n_heads = L.n_heads;
  a.ratio = L.ratio;
  a.k = L.topk_idx ? L.k : 0;
  a.has_topk = L.topk_idx != nullptr;
  a.window = L.window;
  a.n_max = L.max_context / L.ratio;
  a.rows_per_split = p.rows_per_split;
  a.splits = p.splits;
  a.hgp = p.head_groups * 16;
  a.cu_q = L.cu_q;
  a.q_pos = L.q_pos;
  a.q = L.q;
  a.topk = L.topk_idx;
  a.kv = to_dev(L.kv);
  a.swa = to_dev(L.swa);
  a.sm_scale2 = L.softmax_scale * kLog2e;
  const size_t slots = (size_t)L.total_q * p.splits * p.head_groups * 16;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + ((slots * dim * sizeof(float) + 255) & ~(size_t)255));
  const dim3 grid(p.splits, p.head_groups, L.total_q);
  switch (L.kv->dtype) {
    case CSA_FP8_E4M3: launch_q<CSA_FP8_E4M3>(a, L.q_dtype, dim, grid, stream); break;
    case CSA_BF16: launch_q<CSA_BF16>(a, L.q_dtype, dim, grid, stream); break;
    default: launch_q<CSA_F32>(a, L.q_dtype, dim, grid, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs m{};
  m.n_heads = L.n_heads;
  m.splits = p.splits;
  m.hgp = a.hgp;
  m.dim = dim;
  m.rope_dims = L.rope_dims;
  m.rope = make_rope_table(L.rope_base, L.rope_dims);
  m.q_pos = L.q_pos;
  m.part_o = a.part_o;
  m.part_ml = a.part_ml;
  m.out = L.out;
  m.lse = L.lse;
  hipLaunchKernelGGL(attn_merge, dim3((L.n_heads + 3) / 4, L.total_q), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace csa
