// Sparse multi-query attention with K = V over top-k compressed entries plus the sliding
// window, followed by inverse RoPE at the query position.
//
// [vLLM-V4] section 2: keys and values are the same vectors (2x saving); queries attend to
// the top-k compressed tokens plus 128 uncompressed window tokens.  [vLLM-V4] appendix, why
// inverse RoPE: with v_n = k_n = R_n k the output must be multiplied by R_m^{-1}, leaving
// R_{n-m}.  [vLLM-V4] appendix, exact k values: c128a attends to every entry (top-k = 8192).
//
// Kernel 1 (attn_partial), grid (row split, 16-head group, query), 4 waves:
//   every wave owns the 16 heads of its group and walks its own 32-row blocks of the split
//   (blocks w, w+4, ...), keeping a private online softmax and output; the four waves are
//   merged through LDS at the end and one partial (m, l, O) per head leaves the workgroup.
//   Per 32-row block (two 16-row tiles T0, T1):
//     QK : S^T[16 rows x 16 heads] = R_T . Q^T on MFMA 16x16x32 bf16.  Lane (r, g) holds row
//          r of the tile, 8 dims per k-step, loaded straight from HBM (no LDS): the row
//          gather and the MFMA operand layout coincide.
//     PV : O^T[dims x heads] += R^T . P^T.  The transposed operand R^T is produced on the
//          matrix cores by a "selection" MFMA, R_T . Sel_h with Sel_h a 0/1 matrix picking 16
//          of the 32 dims of a k-step: its output layout (4 rows x 1 dim per lane) is exactly
//          the A layout PV needs, with rows of T0 in slots 0-3 and rows of T1 in slots 4-7.
//          P^T comes straight from the QK output registers in the same row order.  P is split
//          into bf16 hi + lo parts (two MFMAs) so PV keeps ~16 significant bits.
//   fp8 rows (code * per-row scale): codes widen exactly to bf16; the scale multiplies the
//   logit and P.  float32 rows / queries are split hi + lo as well.
// Kernel 2 (attn_merge), grid (16-head group, query): combines the splits by their softmax
//   statistics, normalises, applies R_t^{-1} to the last rope_dims dims (angles in float64)
//   and writes out / lse.
#include "common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplits = 256;

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

// Dimension held in slot j of lane group g at k-step ks.
template <int DT>
__device__ __forceinline__ int dim_of_slot(int ks, int g, int j) {
  if (DT == CSA_FP8_E4M3) return 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) + j;
  return 32 * ks + 8 * g + j;
}

__device__ __forceinline__ bf16x8 f32x8_to_bf16(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

// One 16-row tile as seen by lane (r, g): row r's slots for every k-step.
template <int DT, int DIM>
struct Tile {
  static constexpr int NKS = DIM / 32;
  static constexpr int NREG = DT == CSA_FP8_E4M3 ? NKS / 2 : (DT == CSA_BF16 ? NKS : 1);
  uint4 d[NREG];
  const float* f32row;  // float32 rows are re-read per k-step instead of held in registers

  __device__ __forceinline__ void load(const void* rows, int64_t prow, bool valid, int g) {
    if (DT == CSA_F32) {
      f32row = valid ? (const float*)rows + prow * DIM : nullptr;
      return;
    }
#pragma unroll
    for (int i = 0; i < NREG; ++i) d[i] = make_uint4(0, 0, 0, 0);
    if (!valid) return;
    if (DT == CSA_FP8_E4M3) {
      const uint8_t* base = (const uint8_t*)rows + prow * DIM + 16 * g;
#pragma unroll
      for (int kp = 0; kp < NREG; ++kp) d[kp] = *(const uint4*)(base + 64 * kp);
    } else {
      const uint16_t* base = (const uint16_t*)rows + prow * DIM + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NREG; ++ks) d[ks] = *(const uint4*)(base + 32 * ks);
    }
  }

  // bf16 operand for k-step ks (exact for bf16 and fp8 rows); lo = residual for float32 rows.
  __device__ __forceinline__ void frag(int ks, int g, bf16x8& hi, bf16x8& lo) const {
    if (DT == CSA_BF16) {
      hi = __builtin_bit_cast(bf16x8, d[ks]);
    } else if (DT == CSA_FP8_E4M3) {
      const uint4 v = d[ks >> 1];
      const uint32_t w0 = (ks & 1) ? v.z : v.x, w1 = (ks & 1) ? v.w : v.y;
      float x[8];
      fp8x2_to_f32<false>(w0, x[0], x[1]);
      fp8x2_to_f32<true>(w0, x[2], x[3]);
      fp8x2_to_f32<false>(w1, x[4], x[5]);
      fp8x2_to_f32<true>(w1, x[6], x[7]);
      hi = f32x8_to_bf16(x);
    } else {
      float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (f32row) {
        const float4 a = *(const float4*)(f32row + 32 * ks + 8 * g);
        const float4 b = *(const float4*)(f32row + 32 * ks + 8 * g + 4);
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
__global__ __launch_bounds__(256, 1) void attn_partial(Args a) {
  constexpr int NKS = DIM / 32;
  constexpr bool ROW_LO = DT == CSA_F32;
  constexpr bool Q_LO = QDT == CSA_F32;
  __shared__ float o_sh[16][DIM + 4];
  __shared__ float m_sh[4][16], l_sh[4][16];

  const int s = blockIdx.x, hg = blockIdx.y, qi = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ln = lane & 15, lg = lane >> 4;
  const int b = seq_of(a.cu_q, a.batch, qi);
  const int t = a.q_pos[qi];
  const int n_vis = min((t + 1) / a.ratio, a.n_max);
  const int n_c = a.has_topk ? a.k : n_vis;
  const int n_w = min(a.window, t + 1);
  const int n_rows = n_c + n_w;
  const int r_begin = s * a.rows_per_split;
  const int r_end = min(r_begin + a.rows_per_split, n_rows);
  const int H = a.n_heads;

  // Q^T as the B operand: lane (head ln, group lg) holds q[h][dim_of_slot(ks, lg, 0..7)].
  bf16x8 qb[NKS], qb_lo[Q_LO ? NKS : 1];
  {
    const int h = 16 * hg + ln;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int d0 = dim_of_slot<DT>(ks, lg, 0);
      if (QDT == CSA_BF16) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (h < H) v = *(const uint4*)((const uint16_t*)a.q + ((int64_t)qi * H + h) * DIM + d0);
        qb[ks] = __builtin_bit_cast(bf16x8, v);
      } else {
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (h < H) {
          const float* src = (const float*)a.q + ((int64_t)qi * H + h) * DIM + d0;
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = src[i];
        }
        qb[ks] = f32x8_to_bf16(x);
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = x[i] - (float)qb[ks][i];
        if constexpr (Q_LO) qb_lo[ks] = f32x8_to_bf16(r);
      }
    }
  }
  // Sel_h as the B operand: slot (lg, j) -> output column 8 (lg - 2h) + j for lg in {2h, 2h+1}.
  bf16x8 sel[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sel[hh][j] = (__bf16)((lg == 2 * hh + (ln >> 3) && j == (ln & 7)) ? 1.0f : 0.0f);
  }

  f32x4 o[NKS][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    o[ks][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    o[ks][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m_run = -INFINITY, l_run = 0.f;

  for (int row0 = r_begin + 32 * wv; row0 < r_end; row0 += 128) {
    // ---- gather: lane (ln, lg) loads row ln of tile T0 (rows row0..+15) and T1 (+16..+31)
    Tile<DT, DIM> tile[2];
    float rscale[2];
    int rvalid[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const int pos = row0 + 16 * T + ln;
      bool valid = false;
      const DevCache* c = &a.kv;
      int64_t prow = 0;
      if (pos < r_end) {
        if (pos < n_c) {
          const int j = a.has_topk ? a.topk[(int64_t)qi * a.k + pos] : pos;
          if (j >= 0 && j < n_vis) {
            valid = true;
            prow = phys_row(a.kv, b, j);
          }
        } else {
          const int p = t - n_w + 1 + (pos - n_c);
          valid = true;
          c = &a.swa;
          prow = phys_row(a.swa, b, p);
        }
      }
      tile[T].load(c->rows, prow, valid, lg);
      rscale[T] = valid ? (DT == CSA_FP8_E4M3 ? c->scales[prow] : 1.0f) : 0.f;
      rvalid[T] = valid;
    }

    // ---- S^T = R . Q^T
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        bf16x8 rh, rl;
        tile[T].frag(ks, lg, rh, rl);
        sacc[T] = mfma16x16x32(rh, qb[ks], sacc[T]);
        if constexpr (Q_LO) sacc[T] = mfma16x16x32(rh, qb_lo[ks], sacc[T]);
        if constexpr (ROW_LO) sacc[T] = mfma16x16x32(rl, qb[ks], sacc[T]);
      }
    }

    // ---- online softmax; lane (head ln, lg) holds rows 4 lg + jj of T0 and T1
    float z[2][4], sc[2][4];
    float mloc = -INFINITY;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int src = 4 * lg + jj;
        const int v = __shfl(rvalid[T], src, kWave);
        sc[T][jj] = __shfl(rscale[T], src, kWave);
        z[T][jj] = v ? sacc[T][jj] * sc[T][jj] * a.sm_scale2 : -INFINITY;
        mloc = fmaxf(mloc, z[T][jj]);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float m_new = fmaxf(m_run, mloc);
    if (m_new == -INFINITY) continue;  // every row so far is padding (uniform per head)
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    m_run = m_new;
    float pv[8];
    float psum = 0.f;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float p = (z[T][jj] == -INFINITY) ? 0.f : exp2f(z[T][jj] - m_new);
        psum += p;
        pv[4 * T + jj] = p * sc[T][jj];
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      o[ks][0] *= alpha;
      o[ks][1] *= alpha;
    }
    bf16x8 p_hi = f32x8_to_bf16(pv), p_lo;
    {
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = pv[i] - (float)p_hi[i];
      p_lo = f32x8_to_bf16(r);
    }

    // ---- O^T += R^T . P^T, R^T made by the selection MFMA
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 r0h, r0l, r1h, r1l;
      tile[0].frag(ks, lg, r0h, r0l);
      tile[1].frag(ks, lg, r1h, r1l);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 c0 = mfma16x16x32(r0h, sel[hh], zero);
        const f32x4 c1 = mfma16x16x32(r1h, sel[hh], zero);
        bf16x8 at;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          at[jj] = (__bf16)c0[jj];
          at[4 + jj] = (__bf16)c1[jj];
        }
        o[ks][hh] = mfma16x16x32(at, p_hi, o[ks][hh]);
        o[ks][hh] = mfma16x16x32(at, p_lo, o[ks][hh]);
        if constexpr (ROW_LO) {
          const f32x4 d0 = mfma16x16x32(r0l, sel[hh], zero);
          const f32x4 d1 = mfma16x16x32(r1l, sel[hh], zero);
          bf16x8 al;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            al[jj] = (__bf16)d0[jj];
            al[4 + jj] = (__bf16)d1[jj];
          }
          o[ks][hh] = mfma16x16x32(al, p_hi, o[ks][hh]);
        }
      }
    }
  }

  // ---- merge the four waves of the workgroup through LDS
  float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (lg == 0) {
    m_sh[wv][ln] = m_run;
    l_sh[wv][ln] = l_tot;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, m_sh[w][ln]);
  const float f = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);
  for (int w = 0; w < 4; ++w) {
    if (wv == w) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int m = 4 * lg + jj;  // output column of the selection = row of O^T
            const int d = dim_of_slot<DT>(ks, 2 * hh + (m >> 3), m & 7);
            const float v = f * o[ks][hh][jj];
            if (w == 0) o_sh[ln][d] = v; else o_sh[ln][d] += v;
          }
        }
      }
    }
    __syncthreads();
  }
  const int64_t pbase = ((int64_t)qi * a.splits + s) * a.hgp + 16 * hg;
  for (int i = threadIdx.x; i < 16 * DIM; i += 256) {
    const int h = i / DIM, d = i - h * DIM;
    a.part_o[(pbase + h) * DIM + d] = o_sh[h][d];
  }
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float Mh = -INFINITY;
    for (int w = 0; w < 4; ++w) Mh = fmaxf(Mh, m_sh[w][h]);
    float L = 0.f;
    for (int w = 0; w < 4; ++w)
      if (m_sh[w][h] != -INFINITY) L += exp2f(m_sh[w][h] - Mh) * l_sh[w][h];
    a.part_ml[(pbase + h) * 2 + 0] = Mh;
    a.part_ml[(pbase + h) * 2 + 1] = L;
  }
}

struct MergeArgs {
  int n_heads, splits, hgp, dim, rope_dims;
  double rope_base;
  const int32_t* q_pos;
  const float* part_o;
  const float* part_ml;
  float* out;
  float* lse;
};

__global__ __launch_bounds__(256) void attn_merge(MergeArgs a) {
  __shared__ float wgt[kMaxSplits][16];
  __shared__ float cs[64], sn[64];
  const int hg = blockIdx.x, qi = blockIdx.y, tid = threadIdx.x;
  const int t = a.q_pos[qi];
  if (tid < a.rope_dims / 2) rope_cos_sin(-(double)t, tid, a.rope_dims, a.rope_base, cs[tid], sn[tid]);
  const int64_t qbase = (int64_t)qi * a.splits;
  if (tid < 16) {
    const int h = tid;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.part_ml[((qbase + s) * a.hgp + 16 * hg + h) * 2]);
    float L = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float m = a.part_ml[((qbase + s) * a.hgp + 16 * hg + h) * 2];
      const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
      wgt[s][h] = w;
      L += w * a.part_ml[((qbase + s) * a.hgp + 16 * hg + h) * 2 + 1];
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    for (int s = 0; s < a.splits; ++s) wgt[s][h] *= inv;
    const int hh = 16 * hg + h;
    if (a.lse && hh < a.n_heads)
      a.lse[(int64_t)qi * a.n_heads + hh] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  const int half = a.dim / 2;
  const int rope0 = a.dim - a.rope_dims;
  for (int i = tid; i < 16 * half; i += 256) {
    const int h = i / half, d0 = 2 * (i - h * half);
    const int hh = 16 * hg + h;
    if (hh >= a.n_heads) continue;
    float v0 = 0.f, v1 = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float w = wgt[s][h];
      const float2 p = *(const float2*)(a.part_o + ((qbase + s) * a.hgp + hh) * a.dim + d0);
      v0 = fmaf(w, p.x, v0);
      v1 = fmaf(w, p.y, v1);
    }
    if (d0 >= rope0) {
      const int pi = (d0 - rope0) >> 1;
      const float c = cs[pi], sv = sn[pi];
      const float r0 = v0 * c - v1 * sv, r1 = v0 * sv + v1 * c;
      v0 = r0;
      v1 = r1;
    }
    *(float2*)(a.out + ((int64_t)qi * a.n_heads + hh) * a.dim + d0) = make_float2(v0, v1);
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
  bpw = std::min(bpw, blocks32);
  int64_t splits = (blocks32 + bpw - 1) / bpw;
  if (splits > kMaxSplits) {
    bpw = (blocks32 + kMaxSplits - 1) / kMaxSplits;
    splits = (blocks32 + bpw - 1) / bpw;
  }
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
  m.rope_base = (double)L.rope_base;
  m.q_pos = L.q_pos;
  m.part_o = a.part_o;
  m.part_ml = a.part_ml;
  m.out = L.out;
  m.lse = L.lse;
  hipLaunchKernelGGL(attn_merge, dim3(p.head_groups, L.total_q), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace csa
