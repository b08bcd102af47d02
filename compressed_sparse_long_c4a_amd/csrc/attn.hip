// Sparse multi-query attention with K = V over top-k compressed entries plus the sliding
// window, followed by inverse RoPE at the query position.
//
// [vLLM-V4] section 2: keys and values are the same vectors (2x saving); queries attend to
// the top-k compressed tokens plus 128 uncompressed window tokens.  [vLLM-V4] appendix, why
// inverse RoPE: with v_n = k_n = R_n k the output must be multiplied by R_m^{-1}, leaving
// R_{n-m}.  [vLLM-V4] appendix, exact k values: c128a attends to every entry (top-k = 8192).
//
// Three partial kernels, one per row / query format: attn_partial_w (bf16 rows, bf16 queries)
// and attn_partial_fp8 (fp8 rows, bf16 queries) are described where they are defined; the
// generic one covers float32 rows or queries:
// Kernel 1 (attn_partial), grid (row split, 16-head group, query).  The addresses (and fp8
//   scales) of the split's rows are resolved once into LDS.  The workgroup's waves are
//   (dq, ri): dq picks a quarter of the row's dimensions (32-dim k-steps, 5/5/4/4 of 18 for
//   576), ri a row group; row group ri takes the 16-row blocks ri, ri + kRG, ... of the split,
//   its four quarter waves in step.  Per block:
//     QK : each quarter wave computes the partial S^T[16 rows x 16 heads] = R . Q^T over its
//          dimensions on MFMA 16x16x32 bf16 (lane (r, g) holds row r, dims 32 ks + 8 g .. +7,
//          loaded straight from HBM; Q^T, the B operand, stays in registers) and publishes it
//          in LDS; after one barrier each wave adds the row group's four partials in the same
//          order, so the four hold identical S.
//     softmax on the accumulators (identical in the four waves): lane (h, g) holds rows
//          4 g .. 4 g + 3 of head h, the B-operand layout of P^T, so P needs no data movement.
//     PV : each wave accumulates O^T[its dims x 16 heads] only.  The bf16 quarter-rows it
//          loaded, written to its LDS tile during QK, are read back transposed with
//          ds_read_b64_tr_b16 (4 rows x 1 dim per lane).  P is split into bf16 hi + lo parts,
//          which fill the two halves of the K = 32 slots of one MFMA 16x16x32 with V^T
//          repeated in both halves: one MFMA per tile computes V^T (P_hi + P_lo), so PV keeps
//          ~16 significant bits of P at the cost of a plain bf16 product.
//   Every row is thus read from memory once per head group, and a wave's state (Q^T and O of
//   its quarter, a ring of prefetched quarter-row tiles) is small enough for two waves per
//   SIMD, whose memory and LDS latencies overlap.
//   The softmax keeps a per-head reference exponent that moves only when a block's maximum
//   exceeds it by more than kSlack (2^kSlack bounds P), so the output rescale is rare.
//   fp8 rows (code * per-row scale): codes widen exactly to bf16; the scale multiplies the
//   logit and P.  float32 rows / queries are split hi + lo as well (a second PV pass over the
//   rows' lo parts).  The row groups' (m, l, O) are merged through LDS at the end, and one
//   partial (m, l, O) per head leaves the workgroup.
// Kernel 2 (attn_merge), grid (4-head group, query), one wave per head: combines the splits
//   by their softmax statistics, normalises, applies R_t^{-1} to the last rope_dims dims
//   (angles formed and reduced in float64) and writes out / lse.  When every query's rows fit
//   one split (prefill chunks: many queries, few rows each) and only float32 output is wanted,
//   kernel 1 finishes the rows itself with the same operations and kernel 2 is not launched.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa {

// Scratch of csa_sparse_attn_decode_noalloc: the split partials live in this array instead of a
// caller workspace.  Each device holds its own copy for the life of the process; host code uses
// only the device address resolved by attn_static_scratch, never the array's name.
static __device__ __align__(256) unsigned char scratch[kAttnStaticScratchBytes];

void* attn_static_scratch(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // (with device `dev` current)
    if (*err != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRowsPerSplit = kAttnRowsCapGeneric;  // most rows a workgroup handles (addresses staged in LDS)
constexpr int kRowsPerSplitF8 = kAttnRowsCapFp8;     // the same for attn_partial_fp8
constexpr int kRG = 2;               // row groups per workgroup (of four quarter waves each)
constexpr int kWaves = 4 * kRG;
constexpr int kThreads = 64 * kWaves;
constexpr float kSlack = 8.0f;       // log2 headroom of P above the softmax reference

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
  int units;        // splits * total_q
  // single split (splits == 1, float32 output only): the workgroup writes the finished rows
  int direct, rope_dims;
  float* out;       // [total_q][n_heads][DIM]
  float* lse;       // [total_q][n_heads] or NULL
  RopeTable rope;
};

// The workgroup's 16 head rows leave as split partials (O relative to 2^M, and (M, L) per
// head) for attn_merge, or -- when the query's rows are one split and only float32 output is
// wanted -- finished: O / L, R_t^{-1} on the last rope_dims dims, and the lse, with the same
// operations attn_merge applies to a single split (its weight 2^(M - M) is exactly 1), so both
// routes give the same bits.  mb: the merged rows in LDS (published); thread h < 16 passes
// head h's (M, L) in (Mh, Lh); hml: LDS for them.  Called by every thread.
template <int DIM, int NT>
__device__ __forceinline__ void store_head_rows(const Args& a, int s, int hg, int qi,
                                                const float (*mb)[DIM + 4], float (*hml)[2],
                                                float Mh, float Lh) {
  auto row4 = [&](int h, int d) { return *(const float4*)&mb[h][d]; };
  const int tid = threadIdx.x;
  if (a.direct) {
    if (tid < 16) {
      hml[tid][0] = Mh;
      hml[tid][1] = Lh;
    }
    __syncthreads();
    const int t = a.q_pos[qi];
    const int rope0 = DIM - a.rope_dims;
    for (int i = tid; i < 16 * DIM / 4; i += NT) {
      const int h = i / (DIM / 4), d = 4 * (i - h * (DIM / 4));
      const int hq = 16 * hg + h;
      if (hq >= a.n_heads) continue;
      const float L = hml[h][1];
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      const float4 v = row4(h, d);
      float4 r = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
      if (d >= rope0) {  // pairs (d, d+1) and (d+2, d+3) by -t theta_i
        float c0, s0, c1, s1;
        rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2], c0, s0);
        rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2 + 1], c1, s1);
        r = make_float4(r.x * c0 - r.y * s0, r.x * s0 + r.y * c0, r.z * c1 - r.w * s1, r.z * s1 + r.w * c1);
      }
      *(float4*)(a.out + ((int64_t)qi * a.n_heads + hq) * DIM + d) = r;
    }
    if (a.lse && tid < 16 && 16 * hg + tid < a.n_heads) {
      const float M = hml[tid][0], L = hml[tid][1];
      a.lse[(int64_t)qi * a.n_heads + 16 * hg + tid] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
    return;
  }
  const int64_t pbase = ((int64_t)qi * a.splits + s) * a.hgp + 16 * hg;
  for (int i = tid; i < 16 * DIM / 4; i += NT) {
    const int h = i / (DIM / 4), d = 4 * (i - h * (DIM / 4));
    *(float4*)(a.part_o + (pbase + h) * DIM + d) = row4(h, d);
  }
  if (tid < 16) {
    a.part_ml[(pbase + tid) * 2 + 0] = Mh;
    a.part_ml[(pbase + tid) * 2 + 1] = Lh;
  }
}

// Workgroup coordinates (split, head group, query) on the 1-D grid: consecutive workgroup ids
// go to the eight XCDs in turn, so the head groups of one (split, query) get ids eight apart --
// they run on the same XCD at about the same time and read the split's rows once from HBM and
// then from that XCD's L2.  Ids past the last unit exit.
__device__ __forceinline__ bool wg_coords(const Args& a, int& s, int& hg, int& qi) {
  const int id = blockIdx.x, x = id & 7, slot = id >> 3;
  const int G = a.hgp / 16;
  const int u = 8 * (slot / G) + x;
  if (u >= a.units) return false;
  hg = slot - G * (slot / G);
  s = u % a.splits;
  qi = u / a.splits;
  return true;
}

// The same for workgroups of four head groups (head-group quad hq).
__device__ __forceinline__ bool wg_coords_hq(const Args& a, int& s, int& hq, int& qi) {
  const int id = blockIdx.x, x = id & 7, slot = id >> 3;
  const int G = a.hgp / 64;
  const int u = 8 * (slot / G) + x;
  if (u >= a.units) return false;
  hq = slot - G * (slot / G);
  s = u % a.splits;
  qi = u / a.splits;
  return true;
}

// One wave writes its 16 head rows (in wb, LDS, written by this wave) finished: O / L, R_t^{-1}
// on the last rope_dims dims, the lse -- the operations attn_merge applies to a single split.
// Lane (head ln, any group) passes head ln's (M, L).
template <int DIM>
__device__ __forceinline__ void store_head_rows_wave(const Args& a, int hg, int qi, const float (*wb)[DIM + 4],
                                                     float M, float L) {
  const int lane = threadIdx.x & 63;
  const int t = a.q_pos[qi];
  const int rope0 = DIM - a.rope_dims;
  for (int i = lane; i < 16 * DIM / 4; i += 64) {
    const int h = i / (DIM / 4), d = 4 * (i - h * (DIM / 4));
    const int hq = 16 * hg + h;
    const float Lh = __shfl(L, h);
    if (hq >= a.n_heads) continue;
    const float inv = Lh > 0.f ? 1.0f / Lh : 0.f;
    const float4 v = *(const float4*)&wb[h][d];
    float4 r = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    if (d >= rope0) {  // pairs (d, d+1) and (d+2, d+3) by -t theta_i
      float c0, s0, c1, s1;
      rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2], c0, s0);
      rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2 + 1], c1, s1);
      r = make_float4(r.x * c0 - r.y * s0, r.x * s0 + r.y * c0, r.z * c1 - r.w * s1, r.z * s1 + r.w * c1);
    }
    *(float4*)(a.out + ((int64_t)qi * a.n_heads + hq) * DIM + d) = r;
  }
  if (a.lse && lane < 16 && 16 * hg + lane < a.n_heads)
    a.lse[(int64_t)qi * a.n_heads + 16 * hg + lane] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

__device__ __forceinline__ bf16x8 f32x8_to_bf16(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}


// One 16-row block as lane (r, g) holds it: dims 32 ks + 8 g .. +7 of row r for each of the
// NKS k-steps.
template <int DT, int NKS>
struct RowTile {
  static constexpr int NREG = DT == CSA_F32 ? 1 : NKS;
  typedef typename std::conditional<DT == CSA_FP8_E4M3, uint2, uint4>::type Word;
  Word d[NREG];
  const float* f32row;  // float32 rows are re-read per k-step instead of held in registers

  // `row` is always a loadable row (padding rows point at a safe row and are masked later).
  __device__ __forceinline__ void load(const char* row, int g) {
    if constexpr (DT == CSA_F32) {
      f32row = (const float*)row + 8 * g;
    } else {
      constexpr int ESZ = DT == CSA_BF16 ? 2 : 1;
      const char* base = row + 8 * g * ESZ;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) d[ks] = *(const Word*)(base + 32 * ks * ESZ);
    }
  }

  // bf16 operand for k-step ks (exact for bf16 and fp8 rows); lo = residual of float32 rows.
  __device__ __forceinline__ void frag(int ks, bf16x8& hi, bf16x8& lo) const {
    if constexpr (DT == CSA_BF16) {
      hi = __builtin_bit_cast(bf16x8, d[ks]);
    } else if constexpr (DT == CSA_FP8_E4M3) {
      hi = fp8x8_to_bf16x8(d[ks].x, d[ks].y);
    } else {
      float x[8];
      {
        const float4 a = *(const float4*)(f32row + 32 * ks);
        const float4 b = *(const float4*)(f32row + 32 * ks + 4);
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

template <int DT, int QDT, int DIM>
__global__ __launch_bounds__(kThreads) void attn_partial(Args a) {
  constexpr int NKS = DIM / 32;        // QK k-steps of a full row
  constexpr int MQ = (NKS + 3) / 4;    // k-steps of the largest quarter
  constexpr bool ROW_LO = DT == CSA_F32;
  constexpr bool Q_LO = QDT == CSA_F32;
  constexpr int ESZ = DT == CSA_F32 ? 4 : (DT == CSA_BF16 ? 2 : 1);
  // byte offset of each row from the main cache's row base (window rows included), so every
  // row address is derived from a kernel argument and the loads are known to be global
  __shared__ int64_t off_sh[kRowsPerSplit];
  __shared__ float scale_sh[kRowsPerSplit];  // row scale (1 for bf16/f32 rows); 0 marks padding
  // each wave's bf16 quarter-rows of its current block (row stride padded by 16 B so the 16
  // rows of a b128 write start in distinct bank quads); the final merge reuses the space as
  // one float32 [16][DIM + 4] buffer
  constexpr int TROW = MQ * 64 + 16;
  constexpr int TILE_BYTES = kWaves * 16 * TROW;
  constexpr int MERGE_BYTES = 16 * (DIM + 4) * 4;
  __shared__ __attribute__((aligned(16))) char tile_sh[TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES];
  __shared__ f32x4 sx_sh[2][kRG][4][64];  // partial S^T of each quarter: [step parity][row group]
  __shared__ float ml_sh[kRG][16][2];
  __shared__ float hml_sh[16][2];  // per head (M, L) of the workgroup

  int s, hg, qi;
  if (!wg_coords(a, s, hg, qi)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: scalar branches below)
  const int ln = lane & 15, lg = lane >> 4;
  // wave (dq, ri): waves 2 dq + ri share a SIMD pairwise with a wave of another quarter size
  const int dq = wv / kRG, ri = wv % kRG;
  const int nkq = NKS / 4 + (dq < NKS % 4 ? 1 : 0);              // k-steps of quarter dq
  const int k0 = dq * (NKS / 4) + min(dq, NKS % 4);               // its first k-step
  const int H = a.n_heads;
  const char* kvbase = (const char*)a.kv.rows;
  const int r_begin = s * a.rows_per_split;

  // ---- loads that need nothing else: the query position, its sequence, the split's list
  // entries (list positions are bounded by k, so they are read before t is known), Q^T
  const int t = a.q_pos[qi];
  const int b = seq_of_wave(a.cu_q, a.batch, qi);
  constexpr int RPT = kRowsPerSplit / kThreads;
  int ent[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int pos = r_begin + min(tid + kThreads * u, a.rows_per_split - 1);
    ent[u] = a.has_topk ? a.topk[(int64_t)qi * a.k + min(pos, a.k - 1)] : pos;
  }
  // Q^T as the B operand of quarter dq: lane (head ln, group lg) holds q[h][32 ks + 8 lg + 0..7]
  bf16x8 qb[MQ], qb_lo[Q_LO ? MQ : 1];
  {
    const int h = 16 * hg + ln;
#pragma unroll
    for (int kk = 0; kk < MQ; ++kk) {
      const int d0 = 32 * min(k0 + kk, NKS - 1) + 8 * lg;
      const bool use = h < H && kk < nkq;  // a short quarter's missing k-step stays zero
      if constexpr (QDT == CSA_BF16) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (use) v = *(const uint4*)((const uint16_t*)a.q + ((int64_t)qi * H + h) * DIM + d0);
        qb[kk] = __builtin_bit_cast(bf16x8, v);
      } else {
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (use) {
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

  const int n_vis = min((t + 1) / a.ratio, a.n_max);
  const int n_c = a.has_topk ? a.k : n_vis;
  const int n_w = min(a.window, t + 1);
  const int n_rows = n_c + n_w;
  // a query without any visible row (no window and no entry yet) attends to nothing
  const int nrows = (n_w > 0 || n_vis > 0) ? max(0, min(a.rows_per_split, n_rows - r_begin)) : 0;
  // padded to whole steps (16 rows per row group); rows_per_split is a multiple of 16 kRG
  const int nrows_p = (nrows + 16 * kRG - 1) / (16 * kRG) * (16 * kRG);

  // ---- resolve the split's rows once: offset and scale; padding rows (up to a whole step)
  // -> a safe row (finite data) with scale 0.  The block-table reads of all of a thread's rows are
  // issued together, then the scale reads.
  if (nrows > 0) {  // (all staged positions are then rows of this query)
    const int64_t swa_off = (int64_t)((uintptr_t)a.swa.rows - (uintptr_t)a.kv.rows);
    const int64_t safe = n_w > 0 ? swa_off + phys_row(a.swa, b, t) * (DIM * ESZ)
                                 : phys_row(a.kv, b, max(n_vis - 1, 0)) * (DIM * ESZ);
    int64_t prow[RPT];
    bool is_kv[RPT], ok[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = tid + kThreads * u;
      const int pos = r_begin + min(i, nrows - 1);
      is_kv[u] = pos < n_c;
      ok[u] = i < nrows && (!is_kv[u] || (ent[u] >= 0 && ent[u] < n_vis));
      prow[u] = is_kv[u] ? (ok[u] ? phys_row(a.kv, b, ent[u]) : 0)
                         : phys_row(a.swa, b, t - n_w + 1 + (pos - n_c));
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = tid + kThreads * u;
      if (i < nrows_p) {
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

  f32x4 o[2 * MQ];  // O^T of quarter dq: dim tile 16 d' .. +15 (d' < 2 nkq) x 16 heads
#pragma unroll
  for (int dt = 0; dt < 2 * MQ; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;  // per head: reference exponent (log2 units), sum of P
  __syncthreads();

  const int steps = nrows_p / (16 * kRG);  // blocks of every row group
  char* wtile = tile_sh + wv * 16 * TROW;
  lds_char* wtile3 = (lds_char*)wtile;
  // lane (row ln, group lg): dims 32 (k0 + kk) + 8 lg .. +7 of its row for each kk < nkq
  typedef typename std::conditional<DT == CSA_FP8_E4M3, uint2, uint4>::type Word;
  struct Tile {
    Word d[DT == CSA_F32 ? 1 : MQ];
    const float* f32row;  // float32 rows are re-read per k-step instead of held in registers
  };
  // Row loads are unconditional (clamped to the last step; with no step at all, row 0 of the
  // cache): the wait counters then keep the next blocks in flight while one is computed.
  auto load_block = [&](int i, Tile& tl) {
    const int bi = ri + kRG * max(0, min(i, steps - 1));
    const int64_t off = steps > 0 ? off_sh[16 * bi + ln] : 0;
    const char* row = kvbase + off + (32 * k0 + 8 * lg) * ESZ;
    if constexpr (DT == CSA_F32) {
      tl.f32row = (const float*)row;
    } else {
#pragma unroll
      for (int kk = 0; kk < MQ; ++kk) {
        // (a missing last k-step of a short quarter reloads the previous one)
        const int kc = kk < nkq ? kk : nkq - 1;
        tl.d[kk] = *(const Word*)(row + 32 * kc * ESZ);
      }
    }
  };
  // bf16 operand of local k-step kk (exact for bf16 and fp8 rows); lo = float32 residual
  auto frag = [&](const Tile& tl, int kk, bf16x8& hi, bf16x8& lo) {
    if constexpr (DT == CSA_BF16) {
      hi = __builtin_bit_cast(bf16x8, tl.d[kk]);
    } else if constexpr (DT == CSA_FP8_E4M3) {
      hi = fp8x8_to_bf16x8(tl.d[kk].x, tl.d[kk].y);
    } else {
      float x[8];
      const int kc = kk < nkq ? kk : nkq - 1;  // (stays inside the row)
      const float4 u0 = *(const float4*)(tl.f32row + 32 * kc);
      const float4 u1 = *(const float4*)(tl.f32row + 32 * kc + 4);
      x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
      x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
      hi = f32x8_to_bf16(x);
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = x[i] - (float)hi[i];
      lo = f32x8_to_bf16(r);
    }
  };
  // V^T fragment of local dim tile dt from the wave's tile: lane (ln, lg) of a 16-lane group
  // supplies row 4 lg + ln / 4, dims 16 dt + 4 (ln % 4) .. +3; the transposing read returns
  // rows 4 lg .. 4 lg + 3 of dim 16 dt + ln.
  auto vt_frag = [&](int dt) -> s16x4 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(wtile3 + (4 * lg + (ln >> 2)) * TROW +
                                                   2 * (16 * dt + 4 * (ln & 3))));
  };
  // (a short quarter also runs its missing last k-step: a zero Q^T fragment adds nothing to S,
  // and the two extra dim tiles accumulate the repeated k-step into O^T tiles never written
  // out; no branch separates a tile's loads from their use)
  auto pv = [&](const bf16x8& pb) {
#pragma unroll
    for (int dt = 0; dt < 2 * MQ; ++dt) {
      const s16x4 at = vt_frag(dt);
      o[dt] = mfma16x16x32(
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(at, at, 0, 1, 2, 3, 0, 1, 2, 3)), pb, o[dt]);
    }
  };

  // One step: row group ri takes its block i; every wave passes the barrier.
  auto step = [&](int i, const Tile& tl) {
    const int par = i & 1;
    // partial S^T = R . Q^T over this quarter; the bf16 quarter-rows go to the wave's tile
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < MQ; ++kk) {
      bf16x8 rh, rl;
      frag(tl, kk, rh, rl);
      *(bf16x8*)(wtile + ln * TROW + 2 * (32 * kk + 8 * lg)) = rh;
      acc = mfma16x16x32(rh, qb[kk], acc);
      if constexpr (Q_LO) acc = mfma16x16x32(rh, qb_lo[kk], acc);
      if constexpr (ROW_LO) acc = mfma16x16x32(rl, qb[kk], acc);
    }
    sx_sh[par][ri][dq][lane] = acc;
    barrier_lds();  // the partials of block i are visible; parity par is not reused before
                    // the next barrier, so one barrier per step suffices
    // the full S^T, summed in quarter order so the four waves hold identical values
    f32x4 sacc = sx_sh[par][ri][0][lane];
#pragma unroll
    for (int d = 1; d < 4; ++d) sacc += sx_sh[par][ri][d][lane];
    // online softmax over the block's rows 4 lg + j (scale 0 marks padding)
    const int row0 = 16 * (ri + kRG * i);
    const float4 rs4 = *(const float4*)&scale_sh[row0 + 4 * lg];
    const float rs[4] = {rs4.x, rs4.y, rs4.z, rs4.w};
    float z[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      z[j] = rs[j] != 0.f ? sacc[j] * rs[j] * a.sm_scale2 : -INFINITY;
      mloc = fmaxf(mloc, z[j]);
    }
    mloc = rows_reduce(mloc, [](float x, float y) { return fmaxf(x, y); });
    // move a head's reference only when this block's maximum exceeds it by more than kSlack
    // (always when it has none yet); P = 2^(z - m_ref) <= 2^kSlack stays far from overflow
    const bool move = mloc > m_ref + kSlack;
    if (__ballot(move)) {
      const float m_new = move ? mloc : m_ref;
      // v_exp_f32 directly: the argument is <= 0, and 2^-inf = 0 covers an empty reference
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 2 * MQ; ++dt) o[dt] *= alpha;
    }
    float pvv[4], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // padding rows give 0 (also while every row so far is padding and m_ref is -inf)
      const float p = z[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[j] - m_ref);
      psum += p;
      pvv[j] = p * rs[j];
    }
    l_run += psum;
    // B operand of PV: k-slots 0-3 of each lane group hold P_hi of its rows 4 lg + j, slots 4-7
    // hold P_lo of the same rows; O^T += [V^T | V^T] . [P_hi ; P_lo]
    bf16x8 pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const __bf16 hi = (__bf16)pvv[j];
      pb[j] = hi;
      pb[4 + j] = (__bf16)(pvv[j] - (float)hi);
    }
    pv(pb);
    if constexpr (ROW_LO) {  // float32 rows: V_lo P_hi through the same tile
#pragma unroll
      for (int kk = 0; kk < MQ; ++kk) {
        bf16x8 rh, rl;
        frag(tl, kk, rh, rl);
        *(bf16x8*)(wtile + ln * TROW + 2 * (32 * kk + 8 * lg)) = rl;
      }
      bf16x8 ph = pb;
#pragma unroll
      for (int j = 0; j < 4; ++j) ph[4 + j] = (__bf16)0.0f;
      pv(ph);
    }
  };

  // A ring of four register tiles: the next three blocks' loads are in flight while one is
  // computed.  The unrolled loop body has no branch, so the wait counters see every tile's
  // loads in order; the last steps (fewer than four) run after it on tiles already loaded.
  // (float32 rows are read inside the step and need no ring.)
  {
    Tile t0, t1, t2, t3;
    load_block(0, t0);
    load_block(1, t1);
    load_block(2, t2);
    load_block(3, t3);
    int i = 0;
    for (; i + 4 <= steps; i += 4) {
      step(i, t0);
      load_block(i + 4, t0);
      step(i + 1, t1);
      load_block(i + 5, t1);
      step(i + 2, t2);
      load_block(i + 6, t2);
      step(i + 3, t3);
      load_block(i + 7, t3);
    }
    if (i < steps) step(i, t0);          // (uniform across the workgroup)
    if (i + 1 < steps) step(i + 1, t1);
    if (i + 2 < steps) step(i + 2, t2);
  }

  // ---- merge the row groups through LDS: per head M = max_g m_g, f_g = 2^(m_g - M)
  const float l_tot = rows_reduce(l_run, [](float x, float y) { return x + y; });
  if (dq == 0 && lg == 0) {
    ml_sh[ri][ln][0] = m_ref;
    ml_sh[ri][ln][1] = l_tot;
  }
  __syncthreads();  // also: every wave is done with its tile (the merge buffer aliases them)
  float M = -INFINITY;
#pragma unroll
  for (int g = 0; g < kRG; ++g) M = fmaxf(M, ml_sh[g][ln][0]);
  const float f = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - M);
  float (*mb)[DIM + 4] = reinterpret_cast<float (*)[DIM + 4]>(tile_sh);
  // row group 0 stores f O of its quarter, the others add theirs in turn
  float* dst = &mb[ln][32 * k0 + 4 * lg];
#pragma unroll
  for (int round = 0; round < kRG; ++round) {
    if (ri == round) {
#pragma unroll
      for (int dt = 0; dt < 2 * MQ; ++dt) {
        if (dt < 2 * nkq) {
          float4 v = make_float4(f * o[dt][0], f * o[dt][1], f * o[dt][2], f * o[dt][3]);
          if (round > 0) {
            const float4 w = *(const float4*)(dst + 16 * dt);
            v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
          }
          *(float4*)(dst + 16 * dt) = v;
        }
      }
    }
    __syncthreads();
  }
  float Mh = -INFINITY, L = 0.f;
  if (tid < 16) {
    const int h = tid;
#pragma unroll
    for (int g = 0; g < kRG; ++g) Mh = fmaxf(Mh, ml_sh[g][h][0]);
#pragma unroll
    for (int g = 0; g < kRG; ++g)
      if (ml_sh[g][h][0] != -INFINITY) L += exp2f(ml_sh[g][h][0] - Mh) * ml_sh[g][h][1];
  }
  store_head_rows<DIM, kThreads>(a, s, hg, qi, mb, hml_sh, Mh, L);
}

// ---- fp8 rows with bf16 queries.  The workgroup's eight waves take one 128-row step at a
// time: wave w computes S^T for one 16-row tile of the step over the full row width, the
// per-head step maximum and then P are exchanged through LDS, and every wave accumulates O^T
// over the step's 128 rows for its own eighth of the dimensions (five or four 16-dim tiles of
// 576), so the partial output leaves the workgroup from registers, with no merge inside it.
// Rows gathered from random blocks arrive after a long latency, so a wave issues the loads of
// its next step's rows as soon as it has staged the current step's in LDS (kRing steps in
// flight: the vector L1 passes one step's rows in less time than the step's work takes, and
// keeping a second step in flight only delayed the first ones' rows), and
// every load of the prologue and of the ring is issued unconditionally (clamped, or pointed at
// one cached row when there is nothing left to load): with no branch around them, the wait
// counters wait for exactly the loads a value needs and the next step's rows stay in flight
// meanwhile.  The dependent trips are: (query position, sequence, list entries, query heads)
// -> block table -> (row scales, then rows).
// The waves stage the fp8 codes they loaded in LDS (two barriers per step: the row buffer is
// free; the tiles' maxima with P against the current softmax reference, and a third when the
// reference moves), read their own rows back for QK, and PV reads them transposed with
// ds_read_b64_tr_b8 (a 16-lane group reads an 8-row x 16-byte block and lane l receives column
// l of the 8 rows), which is exactly the A operand of V^T with K = 32 rows: the MFMA rows of
// the two QK tiles of a 32-row block are interleaved (tile h holds rows 8 (r / 4) + 4 h + r % 4)
// so that after the softmax lane (head j, group g) holds P of rows 8 g .. 8 g + 7 -- the B
// operand -- once the two waves' halves are put together.  P is applied as bf16 hi and lo
// parts in two MFMAs.
constexpr int kF8Waves = 8;
constexpr int kF8Threads = 64 * kF8Waves;
constexpr int kStepF8 = 16 * kF8Waves;  // rows per step: one 16-row QK tile per wave
constexpr int kRing = 1;                // register tiles per wave (steps in flight)
static_assert(kRowsPerSplitF8 % kF8Threads == 0 && kRowsPerSplitF8 % kStepF8 == 0, "fp8 split size");
template <int DIM>
__global__ __launch_bounds__(kF8Threads) void attn_partial_fp8(Args a) {
  constexpr int NSEG = DIM / 64;        // 64-byte segments of a row (two k-steps each)
  constexpr int NDT = DIM / 16;         // 16-dim output tiles
  constexpr int DTW = (NDT + kF8Waves - 1) / kF8Waves;  // most output tiles of one wave
  constexpr int VROW = DIM + 16;        // LDS bytes per staged row
  __shared__ int64_t off_sh[kRowsPerSplitF8];
  __shared__ float scale_sh[kRowsPerSplitF8];  // row scale; 0 marks padding
  __shared__ __attribute__((aligned(16))) char v_sh[kStepF8 * VROW];
  __shared__ uint4 p_sh[kF8Waves][64];         // P of each QK tile, lane-major {4 hi, 4 lo} bf16
  __shared__ float mx_sh[kF8Waves][16];        // per-head maximum logit of each QK tile
  __shared__ float l_sh[kF8Waves][16];         // per-head sum of P of each wave's rows

  int s, hg, qi;
  if (!wg_coords(a, s, hg, qi)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lg = lane >> 4;
  const int ndt = NDT / kF8Waves + (wv < NDT % kF8Waves ? 1 : 0);  // this wave's output tiles
  const int dt0 = wv * (NDT / kF8Waves) + min(wv, NDT % kF8Waves);  // its first
  const int H = a.n_heads;
  const char* kvbase = (const char*)a.kv.rows;
  const int r_begin = s * a.rows_per_split;

  // ---- trip 1 (all unconditional): list entries, query heads, sequence start, position
  constexpr int RPT = kRowsPerSplitF8 / kF8Threads;
  int ent[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int pos = r_begin + min(tid + kF8Threads * u, a.rows_per_split - 1);
    ent[u] = a.has_topk ? a.topk[(int64_t)qi * a.k + min(pos, a.k - 1)] : pos;
  }
  constexpr int QS = DIM + 8;                  // bf16 per staged query row (padded)
  constexpr int QV = 16 * DIM / 8;             // 16-byte pieces of the 16 heads
  constexpr int QP = (QV + kF8Threads - 1) / kF8Threads;
  static_assert(16 * QS * 2 <= (int)sizeof(v_sh), "query tile fits the row buffer");
  uint4 qv[QP];
#pragma unroll
  for (int p = 0; p < QP; ++p) {
    const int i = min(p * kF8Threads + tid, QV - 1);
    const int h = i / (DIM / 8), c = i - h * (DIM / 8);
    qv[p] = *(const uint4*)((const uint16_t*)a.q + ((int64_t)qi * H + min(16 * hg + h, H - 1)) * DIM + 8 * c);
  }
  const int cu_v = seq_load(a.cu_q, a.batch);
  const int t = a.q_pos[qi];
  const int b = seq_pick(a.cu_q, a.batch, qi, cu_v);

  const int n_vis = min((t + 1) / a.ratio, a.n_max);
  const int n_c = a.has_topk ? a.k : n_vis;
  const int n_w = min(a.window, t + 1);
  const int n_rows = n_c + n_w;
  const int nrows = (n_w > 0 || n_vis > 0) ? max(0, min(a.rows_per_split, n_rows - r_begin)) : 0;
  // padded to whole steps (the last one may be partial: rows_per_split is a multiple of 32)
  const int nrows_p = (nrows + kStepF8 - 1) / kStepF8 * kStepF8;
  const int steps = nrows_p / kStepF8;

  // ---- trip 2: the block table gives each staged row's address (the kv or the window cache,
  // picked by pointer, one load either way)
  const int64_t swa_off = (int64_t)((uintptr_t)a.swa.rows - (uintptr_t)a.kv.rows);
  int64_t roff[RPT], prow[RPT];  // row: byte offset from the main cache's row base, index
  bool use[RPT], is_kv[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int i = tid + kF8Threads * u;
    const int pos = r_begin + min(i, max(nrows - 1, 0));
    is_kv[u] = pos < n_c;
    use[u] = i < nrows && (!is_kv[u] || (ent[u] >= 0 && ent[u] < n_vis));
    // logical row in its cache: an entry id, or a window position; clamped into the table
    const int64_t lrow = is_kv[u] ? (int64_t)min(max(ent[u], 0), max(n_vis - 1, 0))
                                  : (int64_t)max(t - n_w + 1 + (pos - n_c), 0);
    // (each field picked on its own: a selected struct would be read per lane from memory)
    const int32_t* bt = is_kv[u] ? a.kv.bt : a.swa.bt;
    const int stride = is_kv[u] ? a.kv.bt_stride : a.swa.bt_stride;
    const int shift = is_kv[u] ? a.kv.rpb_shift : a.swa.rpb_shift;
    const int32_t blk = bt[(int64_t)b * stride + (int32_t)(lrow >> shift)];
    prow[u] = ((int64_t)blk << shift) + (lrow & ((1 << shift) - 1));
    roff[u] = (is_kv[u] ? 0 : swa_off) + prow[u] * DIM;
  }
#pragma unroll
  for (int p = 0; p < QP; ++p) {  // the query tile into LDS (its loads are done by now)
    const int i = p * kF8Threads + tid;
    const int h = i / (DIM / 8), c = i - h * (DIM / 8);
    const uint4 v = 16 * hg + h < H ? qv[p] : make_uint4(0, 0, 0, 0);
    if (i < QV) *(uint4*)&((uint16_t*)v_sh)[h * QS + 8 * c] = v;  // (a compile-time bound)
  }
  // ---- trip 3a: the row scales (issued before the rows, so waiting for them never waits
  // for a row); padding and rejected entries read the first scale and get 0
  float sc[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const float* sp = is_kv[u] ? a.kv.scales : a.swa.scales;
    sc[u] = sp[use[u] ? prow[u] : 0];
  }
  // the first used row of the split stands in for padding rows (finite data, scale 0)
  const int64_t safe_off = __shfl(roff[0], 0);  // (thread 0 holds the split's first row)
  // (slots past the split's rows are written too, and never read: no branch, no wait)
#pragma unroll
  for (int u = 0; u < RPT; ++u) off_sh[tid + kF8Threads * u] = use[u] ? roff[u] : safe_off;
  barrier_lds();  // offsets and the query tile (the scale loads stay in flight)
  // QK runs over the dimensions in the order the rows are loaded: lane group lg of 64-byte
  // segment m holds dims 64 m + 16 lg .. +15 (one 16-byte load), k-step 2 m + e takes the half
  // e of them.  Q^T, the B operand, follows the same order: lane (head ln, group lg) holds
  // q[h][64 m + 16 lg + 8 e + 0..7] for k-step 2 m + e.
  bf16x8 qb[2 * NSEG];
#pragma unroll
  for (int ks = 0; ks < 2 * NSEG; ++ks) {
    const int d0 = 64 * (ks >> 1) + 16 * lg + 8 * (ks & 1);
    qb[ks] = __builtin_bit_cast(bf16x8, *(const uint4*)((const uint16_t*)v_sh + ln * QS + d0));
  }
  // this wave's QK tile: 32-row block kb of the step, interleave hh
  const int kb = wv >> 1, hh = wv & 1;
  const int my_row = 32 * kb + 8 * (ln >> 2) + 4 * hh + (ln & 3);  // step row of QK row ln
  const int srow0 = 32 * kb + 8 * lg + 4 * hh;                      // step rows of P lanes
  char* vrow_w = v_sh + my_row * VROW + 16 * lg;
  struct Tile { uint4 d[NSEG]; };
  // Loads of step i's rows for this wave's tile, in whole lines: piece j of lane l is 16-byte
  // chunk f % CPR of the tile's row f / CPR, f = 64 j + l (a row's chunks in consecutive lanes,
  // so an instruction reads whole 128-byte lines of few rows, which the vector L1 passes ~2.7
  // times faster than 64 bytes of each of 16 rows).  The step stages them in LDS and the wave
  // reads its rows back in the MFMA operand layout.  A step past the last (or none at all)
  // reads the first row of the main cache instead, the same bytes for every wave, so the load
  // is there for the wait counters but costs no memory traffic.
  constexpr int CPR = DIM / 16;
  int lrow_j[NSEG], lofs_j[NSEG];
#pragma unroll
  for (int j = 0; j < NSEG; ++j) {
    const int f = 64 * j + lane, r = f / CPR;
    lrow_j[j] = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
    lofs_j[j] = 16 * (f - r * CPR);
  }
  auto load_step = [&](int i, Tile& tl) {
    const int ib = kStepF8 * max(min(i, steps - 1), 0);
#pragma unroll
    for (int j = 0; j < NSEG; ++j) {
      const int64_t o = off_sh[ib + lrow_j[j]];
      tl.d[j] = load_global16(kvbase + (i < steps ? o : 0) + lofs_j[j]);
    }
  };
  // ---- trip 3b: the rows of the first kRing steps
  Tile ring[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) load_step(r, ring[r]);
#pragma unroll
  for (int u = 0; u < RPT; ++u) scale_sh[tid + kF8Threads * u] = use[u] ? sc[u] : 0.f;
  barrier_lds();  // the scales; every wave has read its Q^T (the row buffer is free)

  f32x4 o[DTW];  // O^T of this wave's dims (tile 16 (dt0 + dt) .. +15 x 16 heads)
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;  // per head: reference exponent (log2 units), this
                                         // wave's share of the sum of P

  // One step over the tile in `tl`, which is refilled with step `next` (or the stand-in row).
  auto step = [&](int i, Tile& tl, int next) {
    const int r0 = kStepF8 * i;
    // rows of the step that exist: a split's last step may hold fewer than kStepF8; its 32-row
    // blocks past them are neither staged, nor multiplied, nor read by PV (their P is 0: the
    // padding rows' scale is 0)
    const int live = nrows - r0;
    const bool my_live = 32 * kb < live;  // (wave-uniform)
    barrier_lds();  // #0: every wave is past the previous step's PV (the row buffer is free)
    if (my_live) {
#pragma unroll
      for (int j = 0; j < NSEG; ++j) *(uint4*)(v_sh + lrow_j[j] * VROW + lofs_j[j]) = tl.d[j];
    }
    load_step(next, tl);
    // S^T of this wave's 16 rows over the full width, two accumulation chains (the rows back
    // from LDS in the operand layout; this wave wrote them)
    f32x4 acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (my_live) {
#pragma unroll
      for (int m = 0; m < NSEG; ++m) {
        const uint4 x = *(const uint4*)(vrow_w + 64 * m);
        acc2[0] = mfma16x16x32(fp8x8_to_bf16x8(x.x, x.y), qb[2 * m], acc2[0]);
        acc2[1] = mfma16x16x32(fp8x8_to_bf16x8(x.z, x.w), qb[2 * m + 1], acc2[1]);
      }
    }
    const f32x4 sacc = acc2[0] + acc2[1];
    const float4 rs4 = *(const float4*)&scale_sh[r0 + srow0];
    const float rs[4] = {rs4.x, rs4.y, rs4.z, rs4.w};
    float z[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      z[j] = rs[j] != 0.f ? sacc[j] * rs[j] * a.sm_scale2 : -INFINITY;
      mloc = fmaxf(mloc, z[j]);
    }
    mloc = rows_reduce(mloc, [](float x, float y) { return fmaxf(x, y); });
    // P of this wave's tile against the reference m_ref, published with the tile's maximum:
    // unless the step's maximum moves the reference (the first step, then rarely), that P is
    // final and one barrier publishes both; when it moves, every wave rescales, recomputes P
    // and passes one more barrier (the decision is the same in every wave)
    auto make_p = [&]() -> float {
      float pvv[4], psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = z[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[j] - m_ref);
        psum += p;
        pvv[j] = p * rs[j];
      }
      bf16x8 hl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const __bf16 hi = (__bf16)pvv[j];
        hl[j] = hi;
        hl[4 + j] = (__bf16)(pvv[j] - (float)hi);
      }
      p_sh[wv][lane] = __builtin_bit_cast(uint4, hl);
      return psum;
    };
    float psum = make_p();
    if (lg == 0) mx_sh[wv][ln] = mloc;
    barrier_lds();  // #1: the tiles' maxima, their P and the staged rows
    float mblk = mx_sh[0][ln];
#pragma unroll
    for (int w = 1; w < kF8Waves; ++w) mblk = fmaxf(mblk, mx_sh[w][ln]);
    // the reference moves only when a step's maximum exceeds it by more than kSlack (always
    // when it has none yet)
    const bool move = mblk > m_ref + kSlack;
    if (__ballot(move)) {
      const float m_new = move ? mblk : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) o[dt] *= alpha;
      psum = make_p();  // (no wave reads P before the barrier below)
      barrier_lds();    // #1b: P against the moved reference
    }
    l_run += psum;
    // O^T += V^T . P^T over the step, one 32-row block at a time (P_hi and P_lo MFMAs)
#pragma unroll
    for (int kh = 0; kh < kF8Waves / 2; ++kh) {
      if (32 * kh >= live) break;  // (uniform across the workgroup)
      const bf16x8 pa = __builtin_bit_cast(bf16x8, p_sh[2 * kh][lane]);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, p_sh[2 * kh + 1][lane]);
      const bf16x8 phi = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
      const bf16x8 plo = {pa[4], pa[5], pa[6], pa[7], pb[4], pb[5], pb[6], pb[7]};
      const char* vt = v_sh + (32 * kh + 8 * lg + (ln >> 1)) * VROW + 16 * dt0 + 8 * (ln & 1);
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        if (dt < ndt) {  // (wave-uniform)
          typedef int v2i __attribute__((ext_vector_type(2)));
          const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i*)(vt + 16 * dt));
          const bf16x8 va = fp8x8_to_bf16x8((uint32_t)raw[0], (uint32_t)raw[1]);
          o[dt] = mfma16x16x32(va, phi, o[dt]);
          o[dt] = mfma16x16x32(va, plo, o[dt]);
        }
      }
    }
  };

  {
    int i = 0;
    for (; i + kRing <= steps; i += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) step(i + r, ring[r], i + r + kRing);
    }
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r)
      if (i + r < steps) step(i + r, ring[r], steps);  // (uniform across the workgroup)
  }

  // ---- per head: the sum of P over the waves' rows (m_ref is the same in every wave)
  const float l_w = rows_reduce(l_run, [](float x, float y) { return x + y; });
  if (lg == 0) l_sh[wv][ln] = l_w;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kF8Waves; ++w) L += l_sh[w][ln];
  const int hq = 16 * hg + ln;  // lane (head ln, group lg): dims 16 (dt0 + dt) + 4 lg .. +3
  if (a.direct) {  // one split: the finished rows, as attn_merge would write them
    if (hq < H) {
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      const int rope0 = DIM - a.rope_dims;
      float* dst = a.out + ((int64_t)qi * H + hq) * DIM;
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        if (dt >= ndt) continue;
        const int d = 16 * (dt0 + dt) + 4 * lg;
        float4 r = make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
        if (d >= rope0) {  // pairs (d, d+1) and (d+2, d+3) by -t theta_i
          float c0, s0, c1, s1;
          rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2], c0, s0);
          rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2 + 1], c1, s1);
          r = make_float4(r.x * c0 - r.y * s0, r.x * s0 + r.y * c0, r.z * c1 - r.w * s1, r.z * s1 + r.w * c1);
        }
        *(float4*)(dst + d) = r;
      }
      if (a.lse && wv == 0 && lg == 0)
        a.lse[(int64_t)qi * H + hq] = L > 0.f ? (m_ref + log2f(L)) * kLn2 : -INFINITY;
    }
    return;
  }
  const int64_t pbase = ((int64_t)qi * a.splits + s) * a.hgp + 16 * hg + ln;
  float* dst = a.part_o + pbase * DIM;
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt) {
    if (dt >= ndt) continue;
    const int d = 16 * (dt0 + dt) + 4 * lg;
    *(float4*)(dst + d) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
  }
  if (wv == 0 && lg == 0) {
    a.part_ml[pbase * 2 + 0] = m_ref;
    a.part_ml[pbase * 2 + 1] = L;
  }
}

// ---- bf16 rows with bf16 queries.  Four waves, one per SIMD, and nothing shared between them
// inside the row loop: wave w takes the 16-row tiles w, w + 4, w + 8, ... of the split for the
// workgroup's 16 heads and, per tile, computes S^T over the full row width (Q^T held in
// registers as the B operand), runs its own online softmax, and accumulates O^T over every
// dimension.  Two measured gfx950 costs shape it:
// * loaded straight into the MFMA operand layout, every load instruction would read 64 bytes of
//   each of 16 rows, a pattern the vector L1 serves at ~15 bytes per clock per compute unit;
//   the rows arrive instead by LDS DMA (global_load_lds_dwordx4), each instruction moving whole
//   128-byte lines of 8 rows (~40 bytes per clock including the operand reads back), into two
//   slots per wave, the next tile's DMA in flight while one is computed;
// * PV needs the rows transposed (V^T: a lane holds four rows of one dimension); a transposing
//   LDS read costs ~25 clocks per KB of the compute unit's LDS and a b128 LDS write ~16, so
//   the matrix cores transpose instead: an MFMA of a 16 x 32 operand block with an identity B
//   operand leaves A[4 g .. 4 g + 3][j] in lane (j, g) -- exactly the V^T operand layout -- as
//   float32 values that convert back to bf16 exactly; two such MFMAs per 32-dim k-step.
// A tile thus costs 18 QK + 36 transpose + 36 PV MFMAs.  With one wave per SIMD a wave holds
// Q^T and the whole O^T of its heads; the waves' (m, l, O) are merged through LDS at the end and
// one partial row per head leaves from registers.
constexpr int kWWaves = 4;

// NKS 16-byte LDS reads, k-step ks from base a(ks % 2) + 1024 (ks / 2), issued in one asm block
// that waits for all of them (so no result register is live while its read is in flight).
typedef unsigned int lds_u32x4 __attribute__((ext_vector_type(4)));
#define CSA_R(i, b, o) "ds_read_b128 %" #i ", %" #b " offset:" #o "\n\t"
template <int NKS>
__device__ __forceinline__ void lds_read_tile(uint4 (&d)[NKS], uint32_t a0, uint32_t a1) {
  static_assert(NKS == 16 || NKS == 18, "row widths of 512 or 576 bf16");
  lds_u32x4 v[18];
  if constexpr (NKS == 18) {
    asm volatile(CSA_R(0, 18, 0) CSA_R(1, 19, 0) CSA_R(2, 18, 1024) CSA_R(3, 19, 1024)
                 CSA_R(4, 18, 2048) CSA_R(5, 19, 2048) CSA_R(6, 18, 3072) CSA_R(7, 19, 3072)
                 CSA_R(8, 18, 4096) CSA_R(9, 19, 4096) CSA_R(10, 18, 5120) CSA_R(11, 19, 5120)
                 CSA_R(12, 18, 6144) CSA_R(13, 19, 6144) CSA_R(14, 18, 7168) CSA_R(15, 19, 7168)
                 CSA_R(16, 18, 8192) CSA_R(17, 19, 8192) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
                   "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]),
                   "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15]), "=&v"(v[16]), "=&v"(v[17])
                 : "v"(a0), "v"(a1)
                 : "memory");
  } else {
    asm volatile(CSA_R(0, 16, 0) CSA_R(1, 17, 0) CSA_R(2, 16, 1024) CSA_R(3, 17, 1024)
                 CSA_R(4, 16, 2048) CSA_R(5, 17, 2048) CSA_R(6, 16, 3072) CSA_R(7, 17, 3072)
                 CSA_R(8, 16, 4096) CSA_R(9, 17, 4096) CSA_R(10, 16, 5120) CSA_R(11, 17, 5120)
                 CSA_R(12, 16, 6144) CSA_R(13, 17, 6144) CSA_R(14, 16, 7168) CSA_R(15, 17, 7168)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
                   "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]),
                   "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
                 : "v"(a0), "v"(a1)
                 : "memory");
  }
#pragma unroll
  for (int k = 0; k < NKS; ++k) d[k] = make_uint4(v[k][0], v[k][1], v[k][2], v[k][3]);
}
#undef CSA_R
constexpr int kWThreads = 64 * kWWaves;
static_assert(kRowsPerSplit % kWThreads == 0 && kRowsPerSplit % (16 * kWWaves) == 0, "split size");
template <int DIM, bool HG4>
__global__ __launch_bounds__(kWThreads) void attn_partial_w(Args a) {
  constexpr int NKS = DIM / 32;         // k-steps of a row
  constexpr int NDT = DIM / 16;         // 16-dim output tiles
  constexpr int MROW = DIM + 4;         // floats per row of the two merge buffers
  constexpr int RB = 2 * DIM, NL = RB / 128;  // bytes and 128-byte lines of a row
  constexpr int SLOT = 16 * RB + 128;         // LDS bytes of a tile slot
  static_assert(RB % 128 == 0 && 2 * 16 * MROW * 4 <= 2 * kWWaves * SLOT, "slots hold the merge buffers");
  // each staged row as one word: physical row index, bit 31 = a window row (the window cache),
  // bit 30 = padding or a rejected entry (masked; the word still names a loadable row)
  __shared__ uint32_t row_sh[kRowsPerSplit];
  // two tile slots per wave (the rows arrive here by LDS DMA); the final merge reuses the space
  __shared__ __attribute__((aligned(16))) char slot_sh[2 * kWWaves * SLOT];
  __shared__ float hml_sh[16][2];  // per head (M, L) of the workgroup (single-split rows)
  __shared__ float ml_sh[kWWaves][16][2];

  int s, hg, qi;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (HG4) {  // the workgroup's four waves take head groups 4 q .. 4 q + 3
    if (!wg_coords_hq(a, s, hg, qi)) return;
    hg = 4 * hg + wv;
  } else {
    if (!wg_coords(a, s, hg, qi)) return;
  }
  const int ln = lane & 15, lg = lane >> 4;
  const int H = a.n_heads;
  const char* kvbase = (const char*)a.kv.rows;
  const int r_begin = s * a.rows_per_split;

  // ---- trip 1 (all unconditional): list entries, Q^T, sequence start, position
  constexpr int RPT = kRowsPerSplit / kWThreads;
  int ent[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int pos = r_begin + min(tid + kWThreads * u, a.rows_per_split - 1);
    ent[u] = a.has_topk ? a.topk[(int64_t)qi * a.k + min(pos, a.k - 1)] : pos;
  }
  // Q^T as the B operand: lane (head ln, group lg) holds q[h][32 ks + 8 lg .. +7] (heads past
  // the last repeat it; their rows are never stored).  The workgroup's query heads (16, or 64
  // with HG4) come through LDS: loaded in whole lines (a head's 16-byte chunks in consecutive
  // lanes) into the tile slots, free until the first DMA, and read back in the operand layout
  // (loaded straight into the operand layout, every instruction read 64 bytes of each of 16
  // heads, which the vector L1 passes at ~15 B/clk).
  constexpr int NQH = HG4 ? 4 * 16 : 16;  // heads staged
  constexpr int QCH = DIM / 8;            // 16-byte chunks per head
  constexpr int QROWB = 2 * DIM + 16;     // LDS bytes per staged head (padded)
  constexpr int QPT = (NQH * QCH + kWThreads - 1) / kWThreads;
  const int hbase = HG4 ? 16 * (hg - wv) : 16 * hg;  // the workgroup's first head
  uint4 qst[QPT];
#pragma unroll
  for (int p = 0; p < QPT; ++p) {
    const int f = min(p * kWThreads + tid, NQH * QCH - 1);
    const int hh = f / QCH, c = f - hh * QCH;
    const int h = min(hbase + hh, H - 1);
    qst[p] = load_global16((const uint16_t*)a.q + ((int64_t)qi * H + h) * DIM + 8 * c);
  }
  bf16x8 qb[NKS];
  const int cu_v = seq_load(a.cu_q, a.batch);
  const int t = a.q_pos[qi];
  const int b = seq_pick(a.cu_q, a.batch, qi, cu_v);

  const int n_vis = min((t + 1) / a.ratio, a.n_max);
  const int n_c = a.has_topk ? a.k : n_vis;
  const int n_w = min(a.window, t + 1);
  const int n_rows = n_c + n_w;
  const int nrows = (n_w > 0 || n_vis > 0) ? max(0, min(a.rows_per_split, n_rows - r_begin)) : 0;
  const int ntiles = (nrows + 15) / 16;

  // ---- trip 2: the block table gives each staged row's address (the kv or the window cache,
  // picked by pointer, one load either way)
  uint32_t rw[RPT];
  bool use[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int i = tid + kWThreads * u;
    const int pos = r_begin + min(i, max(nrows - 1, 0));
    const bool is_kv = pos < n_c;
    use[u] = i < nrows && (!is_kv || (ent[u] >= 0 && ent[u] < n_vis));
    const int64_t lrow = is_kv ? (int64_t)min(max(ent[u], 0), max(n_vis - 1, 0))
                               : (int64_t)max(t - n_w + 1 + (pos - n_c), 0);
    const int32_t* bt = is_kv ? a.kv.bt : a.swa.bt;
    const int stride = is_kv ? a.kv.bt_stride : a.swa.bt_stride;
    const int shift = is_kv ? a.kv.rpb_shift : a.swa.rpb_shift;
    const int32_t blk = bt[(int64_t)b * stride + (int32_t)(lrow >> shift)];
    const uint32_t prow = ((uint32_t)blk << shift) + (uint32_t)(lrow & ((1 << shift) - 1));
    rw[u] = prow | (is_kv ? 0u : 0x80000000u);
  }
  // the first row of the split stands in for padding rows (finite data, masked)
  const uint32_t safe = (uint32_t)__shfl((int)rw[0], 0) | 0x40000000u;
#pragma unroll
  for (int u = 0; u < RPT; ++u) row_sh[tid + kWThreads * u] = use[u] ? rw[u] : safe;
  static_assert(NQH * QROWB <= (int)sizeof(slot_sh), "the query heads fit the tile slots");
#pragma unroll
  for (int p = 0; p < QPT; ++p) {
    const int f = p * kWThreads + tid;
    const int hh = f / QCH, c = f - hh * QCH;
    if (f < NQH * QCH) *(uint4*)(slot_sh + hh * QROWB + 16 * c) = qst[p];
  }
  barrier_lds();  // the row words and the query heads
  {
    const char* qrow = slot_sh + ((HG4 ? 16 * wv : 0) + ln) * QROWB + 16 * lg;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qb[ks] = *(const bf16x8*)(qrow + 64 * ks);
  }
  barrier_lds();  // every wave has its Q^T: the slots may take rows
  // Q^T lives in the accumulation registers (the MFMA reads its B operand from either file):
  // the ordinary registers then hold O^T and leave room for the PV operands in flight.
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+a"(qb[ks]));

  // this wave's tiles: every tile of the split (HG4), else tiles wv, wv + 4, ...
  const int ntw = HG4 ? ntiles : (ntiles > wv ? (ntiles - wv + kWWaves - 1) / kWWaves : 0);
  auto tile_of = [&](int j) { return HG4 ? j : wv + kWWaves * j; };
  // identity B operands of the transposing MFMAs: B[k][n] = 1 where k = n (I_lo: dims 0-15 of
  // a k-step) or k = n + 16 (I_hi: dims 16-31); lane (n, g) holds B[8 g .. 8 g + 7][n]
  bf16x8 id_lo, id_hi;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    id_lo[e] = (__bf16)(8 * lg + e == ln ? 1.0f : 0.0f);
    id_hi[e] = (__bf16)(8 * lg + e == ln + 16 ? 1.0f : 0.0f);
  }
  // 16 rows as lane (row ln, group lg) holds them: dims 32 ks + 8 lg .. +7 for every k-step
  struct Tile { uint4 d[NKS]; };
  // The rows come through LDS: loaded straight into the operand layout every load instruction
  // would touch 64 bytes of each of 16 rows, a pattern the vector L1 serves at ~15 bytes per
  // clock per compute unit; LDS DMA instructions that each move whole 128-byte lines of 8 rows,
  // read back with ds_read_b128, run at ~40.  Instruction (rg, c) of the wave's tile j moves
  // line c of rows 8 rg .. 8 rg + 7: lane l fetches row 8 rg + l / 8, 16-byte piece
  // (l % 8) ^ (l / 8) of the line, which the DMA writes at 16 l -- piece p of row r lands at
  // piece p ^ (r % 8) of the row's 128-byte place, so the operand reads fall on distinct banks.
  // Past the wave's last tile (or with none at all) the first row of the main cache is moved.
  lds_char* slots = (lds_char*)slot_sh + 2 * wv * SLOT;  // tile j goes to slot j % 2
  const char* swabase = (const char*)a.swa.rows;
  auto dma_tile = [&](int j) __attribute__((always_inline)) {
    const int tile = tile_of(max(min(j, ntw - 1), 0));
    lds_char* slot = slots + (j & 1) * SLOT;
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const uint32_t w = row_sh[16 * tile + 8 * rg + (lane >> 3)];
      const char* base = (w & 0x80000000u) ? swabase : kvbase;
      const char* row = (j < ntw ? base + (int64_t)(w & 0x3FFFFFFFu) * RB : kvbase) + 16 * ((lane & 7) ^ (lane >> 3));
#pragma unroll
      for (int c = 0; c < NL; ++c)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(row + 128 * c),
                                         (__attribute__((address_space(3))) void*)(slot + (rg * NL + c) * 1024),
                                         16, 0, 0);
    }
  };
  // k-step ks of row ln sits at byte 64 ks + 16 lg of the row: line ks / 2 of its place, piece
  // p = (4 (ks % 2) + lg) % 8, stored at piece p ^ (ln % 8); so the reads of even and of odd
  // k-steps each take one base address plus 1024 (ks / 2).  They are issued from one asm block
  // that also waits for them: the compiler cannot tell which slot an LDS DMA writes, and before
  // a plain LDS read of a slot it waits for every DMA in flight (the next tile's too), which
  // would undo the two-tile prefetch; the DMA of this tile is waited for explicitly instead.
  auto read_tile = [&](int j, Tile& tl) __attribute__((always_inline)) {
    const uint32_t slot = (uint32_t)(uintptr_t)(slots + (j & 1) * SLOT);
    const uint32_t rbase = slot + (ln >> 3) * NL * 1024 + (ln & 7) * 128;
    const uint32_t a0 = rbase + (((lg & 7) ^ (ln & 7)) << 4);        // even k-steps
    const uint32_t a1 = rbase + ((((4 + lg) & 7) ^ (ln & 7)) << 4);  // odd k-steps
    lds_read_tile<NKS>(tl.d, a0, a1);
  };

  f32x4 o[NDT];  // O^T: dim tile 16 dt .. +15 x 16 heads
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;  // per head: reference exponent (log2 units), sum of P

  // QK, softmax and P (bf16 hi + lo) of the wave's tile j, rows in tl.  The transposes of the
  // first kLead k-steps are issued first, so the matrix cores run them during the softmax.
  constexpr int kLead = 3;
  auto transposes = [&](const Tile& tl, int ks, f32x4 (&t)[2]) __attribute__((always_inline)) {
    const bf16x8 rk = __builtin_bit_cast(bf16x8, tl.d[ks]);
    t[0] = mfma16x16x32(rk, id_lo, f32x4{0.f, 0.f, 0.f, 0.f});
    t[1] = mfma16x16x32(rk, id_hi, f32x4{0.f, 0.f, 0.f, 0.f});
  };
  auto qk_softmax = [&](int j, const Tile& tl, f32x4 (&tq)[kLead][2]) __attribute__((always_inline)) -> bf16x8 {
    const int row0 = 16 * tile_of(j);
    f32x4 acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      acc2[ks & 1] = mfma16x16x32(__builtin_bit_cast(bf16x8, tl.d[ks]), qb[ks], acc2[ks & 1]);
    const f32x4 sacc = acc2[0] + acc2[1];
#pragma unroll
    for (int ks = 0; ks < kLead; ++ks) transposes(tl, ks, tq[ks]);
    const uint4 rw4 = *(const uint4*)&row_sh[row0 + 4 * lg];
    const uint32_t rws[4] = {rw4.x, rw4.y, rw4.z, rw4.w};
    float z[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      z[jj] = (rws[jj] & 0x40000000u) ? -INFINITY : sacc[jj] * a.sm_scale2;
      mloc = fmaxf(mloc, z[jj]);
    }
    mloc = rows_reduce(mloc, [](float x, float y) { return fmaxf(x, y); });
    // the reference moves only when a tile's maximum exceeds it by more than kSlack
    const bool move = mloc > m_ref + kSlack;
    if (__ballot(move)) {
      const float m_new = move ? mloc : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    bf16x8 pb;  // k-slots 0-3: P_hi of rows 4 lg + j, 4-7: P_lo of the same rows
    float psum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float p = z[jj] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[jj] - m_ref);
      psum += p;
      const __bf16 hi = (__bf16)p;
      pb[jj] = hi;
      pb[4 + jj] = (__bf16)(p - (float)hi);
    }
    l_run += psum;
    return pb;
  };
  // O^T += [V^T | V^T] . [P_hi ; P_lo]; V^T of dims 32 ks .. +15 and 32 ks + 16 .. +31 from the
  // transposing MFMAs (lane (dim n, group g): rows 4 g .. 4 g + 3, exact in bf16), issued kLead
  // k-steps ahead of their use, so the conversions (VALU) of one k-step run while the matrix
  // cores work on later ones: per k-step two transposes, eight VALU, two PV MFMAs.
  auto pv = [&](const Tile& tl, f32x4 (&tq)[kLead][2], const bf16x8& pb) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f32x4 t0 = tq[ks % kLead][0], t1 = tq[ks % kLead][1];
      if (ks + kLead < NKS) transposes(tl, ks + kLead, tq[ks % kLead]);
      bf16x8 vlo, vhi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vlo[e] = vlo[4 + e] = (__bf16)t0[e];
        vhi[e] = vhi[4 + e] = (__bf16)t1[e];
      }
      o[2 * ks] = mfma16x16x32(vlo, pb, o[2 * ks]);
      o[2 * ks + 1] = mfma16x16x32(vhi, pb, o[2 * ks + 1]);
      if (ks + kLead < NKS) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };

  // The wave's own wait counts order its DMA and its LDS reads (no other load of this wave is in
  // flight in the loop): with tile j + 1's DMA issued after tile j's, tile j has landed once at
  // most that many loads are outstanding, and its slot may take tile j + 2 once the operand
  // reads are back (read_tile waits for them).
  constexpr int kVmcnt0 = 0x0F70;
  constexpr int kVmcntTile = 0x0F70 | ((2 * NL) & 15) | (((2 * NL) >> 4) << 14);  // vmcnt(2 NL)
  dma_tile(0);
  dma_tile(1);
  for (int j = 0; j < ntw; ++j) {
    Tile cur;
    __builtin_amdgcn_s_waitcnt(kVmcntTile);
    read_tile(j, cur);  // (its reads are complete when it returns: the slot is free)
    dma_tile(j + 2);
    f32x4 tq[kLead][2];
    const bf16x8 pb = qk_softmax(j, cur, tq);
    pv(cur, tq, pb);
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);  // (the DMAs past the end) before the slots are reused

  if constexpr (HG4) {
    // each wave holds the whole result of its head group: no merge
    const float L = rows_reduce(l_run, [](float x, float y) { return x + y; });
    const int hq = 16 * hg + ln;
    if (a.direct) {
      // the finished rows through the wave's own slots (free now), one wave, the operations
      // of attn_merge for a single split
      float (*wb)[MROW] = reinterpret_cast<float (*)[MROW]>(slot_sh + 2 * wv * SLOT);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *(float4*)&wb[ln][16 * dt + 4 * lg] = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      store_head_rows_wave<DIM>(a, hg, qi, wb, m_ref, L);
      return;
    }
    const int64_t pbase = ((int64_t)qi * a.splits + s) * a.hgp + hq;
    float* dst = a.part_o + pbase * DIM;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *(float4*)(dst + 16 * dt + 4 * lg) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (lg == 0) {
      a.part_ml[pbase * 2 + 0] = m_ref;
      a.part_ml[pbase * 2 + 1] = L;
    }
    return;
  }

  // ---- merge the waves: per head M = max_w m_w, f_w = 2^(m_w - M).  Each wave writes f_w O_w
  // to its own 16 x DIM buffer (the tile slots, free now, hold exactly four), then every thread
  // sums the four buffers for its share of the 16 heads' rows, which leave in full lines.
  const float l_w = rows_reduce(l_run, [](float x, float y) { return x + y; });
  if (lg == 0) {
    ml_sh[wv][ln][0] = m_ref;
    ml_sh[wv][ln][1] = l_w;
  }
  __syncthreads();  // also: every wave is done with its slots (the merge buffers alias them)
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWWaves; ++w) M = fmaxf(M, ml_sh[w][ln][0]);
  const float f = m_ref == -INFINITY ? 0.f : exp2f(m_ref - M);
  typedef float WaveRows[16][MROW];
  static_assert(kWWaves * sizeof(WaveRows) <= sizeof(slot_sh), "the slots hold the four wave buffers");
  WaveRows* mb4 = reinterpret_cast<WaveRows*>(slot_sh);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    *(float4*)&mb4[wv][ln][16 * dt + 4 * lg] = make_float4(o[dt][0] * f, o[dt][1] * f, o[dt][2] * f, o[dt][3] * f);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kWWaves; ++w)
    if (ml_sh[w][ln][0] != -INFINITY) L += exp2f(ml_sh[w][ln][0] - M) * ml_sh[w][ln][1];
  __syncthreads();
  constexpr int C4 = DIM / 4;  // float4 columns of a row
  const int64_t pbase0 = ((int64_t)qi * a.splits + s) * a.hgp + 16 * hg;
  for (int i = tid; i < 16 * C4; i += kWThreads) {
    const int h = i / C4, c = 4 * (i - h * C4);
    float4 v = *(const float4*)&mb4[0][h][c];
#pragma unroll
    for (int w = 1; w < kWWaves; ++w) {
      const float4 x = *(const float4*)&mb4[w][h][c];
      v = make_float4(v.x + x.x, v.y + x.y, v.z + x.z, v.w + x.w);
    }
    if (a.direct) *(float4*)&mb4[0][h][c] = v;  // (the element this thread read)
    else *(float4*)(a.part_o + (pbase0 + h) * DIM + c) = v;
  }
  if (a.direct) {
    // one split: the finished rows (normalised, R_t^{-1}, lse) by every thread through LDS, with
    // the operations attn_merge applies to a single split
    __syncthreads();
    store_head_rows<DIM, kWThreads>(a, s, hg, qi, mb4[0], hml_sh, M, L);
    return;
  }
  if (wv == 0 && lg == 0) {
    a.part_ml[(pbase0 + ln) * 2 + 0] = M;
    a.part_ml[(pbase0 + ln) * 2 + 1] = L;
  }
}

struct MergeArgs {
  int n_heads, splits, hgp, dim, rope_dims;
  const int32_t* q_pos;
  const float* part_o;
  const float* part_ml;
  float* out;
  float* lse;
  uint8_t* out_fp8;
  float* out_scales;
  RopeTable rope;
};

// One wave per (query, head): split weights from the partial statistics, weighted sum of the
// partial outputs, normalisation and R_t^{-1} on the last rope_dims dims; the row leaves as
// float32 and/or as fp8 codes with one scale (amax / 448, from a wave max: [vLLM-V4] section 3
// part 2, second fusion, inverse RoPE + fp8 quantisation for the output projection).  Each lane owns the
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
  // (m, l) of split lane (the first 64 splits) first, then the partial rows of the first round:
  // one trip; rounds hold only existing splits (the condition is uniform)
  const float2 ml0 = lane < a.splits ? *(const float2*)&ml[lane * mls] : make_float2(-INFINITY, 0.f);
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kMergeRound; ++u) {
      if (s0 + u < a.splits) {
        const int64_t sb = (int64_t)(s0 + u) * stride4;
#pragma unroll
        for (int j = 0; j < kMergeCols; ++j) v[u][j] = src[sb + col[j]];
      }
    }
  };
  load_round(0);
  const int t = a.q_pos[qi];

  // M = max_s m_s (log2 units), L = sum_s 2^(m_s - M) l_s
  float M = ml0.x;
  for (int s = 64 + lane; s < a.splits; s += 64) M = fmaxf(M, ml[s * mls]);
  M = wave_max(M);
  float L = (ml0.x == -INFINITY) ? 0.f : exp2f(ml0.x - M) * ml0.y;
  for (int s = 64 + lane; s < a.splits; s += 64) {
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
      const float m = s0 == 0 ? ml0.x : s < a.splits ? ml[s * mls] : -INFINITY;
      wl = (m == -INFINITY) ? 0.f : exp2f(m - M);
    }
#pragma unroll
    for (int u = 0; u < kMergeRound; ++u) {
      if (s0 + u >= a.splits) break;  // (uniform)
      const float w =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), (s0 & 63) + u));
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
  const int64_t row = (int64_t)qi * a.n_heads + h;
  float4 r[kMergeCols];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kMergeCols; ++j) {
    r[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane + 64 * j >= dim4) continue;
    const int d = 4 * (lane + 64 * j);
    r[j] = make_float4(acc[j].x * inv, acc[j].y * inv, acc[j].z * inv, acc[j].w * inv);
    if (d >= rope0) {  // pairs (d, d+1) and (d+2, d+3) by -t theta_i
      float c0, s0, c1, s1;
      rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2], c0, s0);
      rope_cos_sin(-(double)t, a.rope.theta[(d - rope0) / 2 + 1], c1, s1);
      r[j] = make_float4(r[j].x * c0 - r[j].y * s0, r[j].x * s0 + r[j].y * c0,
                         r[j].z * c1 - r[j].w * s1, r[j].z * s1 + r[j].w * c1);
    }
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(r[j].x), fabsf(r[j].y)), fmaxf(fabsf(r[j].z), fabsf(r[j].w))));
    if (a.out) *(float4*)(a.out + row * a.dim + d) = r[j];
  }
  if (a.out_fp8) {
    amax = wave_max(amax);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < kMergeCols; ++j) {
      if (lane + 64 * j >= dim4) continue;
      const int d = 4 * (lane + 64 * j);
      const uint32_t codes = (uint32_t)f32_to_fp8(r[j].x / scale) | ((uint32_t)f32_to_fp8(r[j].y / scale) << 8) |
                             ((uint32_t)f32_to_fp8(r[j].z / scale) << 16) | ((uint32_t)f32_to_fp8(r[j].w / scale) << 24);
      *(uint32_t*)(a.out_fp8 + row * a.dim + d) = codes;
    }
    if (lane == 0) a.out_scales[row] = scale;
  }
}

template <int DT, int QDT, int DIM>
void launch_partial(const Args& args, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_partial<DT, QDT, DIM>), grid, dim3(kThreads), 0, stream, args);
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

template <>
void launch_q<CSA_BF16>(const Args& args, int qdt, int dim, dim3 grid, hipStream_t stream) {
  if (qdt == CSA_BF16) {
    // one split per query with head groups in fours and enough queries to fill the chip
    // (chunked prefill): each wave takes one head group over all of the query's rows, so the
    // four waves share the row addresses and no merge is needed; otherwise the waves split the
    // rows of one head group
    const bool hg4 = args.splits == 1 && args.hgp % 64 == 0 && (int64_t)args.units * (args.hgp / 64) >= 256;
    if (hg4) {
      const dim3 g4((unsigned)(8 * (int64_t)(args.hgp / 64) * ((args.units + 7) / 8)));
      if (dim == 576) hipLaunchKernelGGL((attn_partial_w<576, true>), g4, dim3(kWThreads), 0, stream, args);
      else hipLaunchKernelGGL((attn_partial_w<512, true>), g4, dim3(kWThreads), 0, stream, args);
    } else {
      if (dim == 576) hipLaunchKernelGGL((attn_partial_w<576, false>), grid, dim3(kWThreads), 0, stream, args);
      else hipLaunchKernelGGL((attn_partial_w<512, false>), grid, dim3(kWThreads), 0, stream, args);
    }
  } else {
    launch_dim<CSA_BF16, CSA_F32>(args, dim, grid, stream);
  }
}

template <>
void launch_q<CSA_FP8_E4M3>(const Args& args, int qdt, int dim, dim3 grid, hipStream_t stream) {
  if (qdt == CSA_BF16) {
    if (dim == 576) hipLaunchKernelGGL((attn_partial_fp8<576>), grid, dim3(kF8Threads), 0, stream, args);
    else hipLaunchKernelGGL((attn_partial_fp8<512>), grid, dim3(kF8Threads), 0, stream, args);
  } else {
    // (fp8 rows with f32 queries: the generic kernel on the XCD-grouped grid)
    const dim3 g1((unsigned)(8 * (int64_t)(args.hgp / 16) * ((args.units + 7) / 8)));
    launch_dim<CSA_FP8_E4M3, CSA_F32>(args, dim, g1, stream);
  }
}

}  // namespace

AttnPlan attn_plan(int total_q, int n_heads, int ratio, int has_topk, int k, int max_context,
                   int window, int rows_cap) {
  AttnPlan p{};
  const int64_t n_max = max_context / ratio;
  p.max_rows = (has_topk ? (int64_t)k : n_max) + std::min<int64_t>(window, max_context);
  p.head_groups = (n_heads + 15) / 16;
  const int64_t blocks32 = std::max<int64_t>(1, (p.max_rows + 31) / 32);
  const int64_t units = (int64_t)total_q * p.head_groups;
  // aim at one workgroup per compute unit (256 CUs).  The generic kernel's splits are whole
  // numbers of 128-row blocks; the fp8-row kernel's are cut at 32 rows (its last step may be
  // partial: the 32-row blocks past the split's rows are skipped), so that e.g. 4 queries x 8
  // head groups x 2,176 rows take 8 splits of 288 rows on 256 compute units, not 6 of 384 on 192
  const int64_t sb = rows_cap == kAttnRowsCapFp8 ? 1 : 4;  // 32-row blocks per unit of a split
  int64_t bpw = std::max<int64_t>(sb, (blocks32 * units + 255) / 256);
  bpw = std::min<int64_t>((std::min(bpw, blocks32) + sb - 1) / sb * sb, rows_cap / 32);
  // (max_rows <= kAttnMaxRows keeps splits <= 512 and the partial workspace finite)
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
  // one split and float32 output only: the partial kernel writes the finished rows itself
  a.direct = p.splits == 1 && L.out != nullptr && L.out_fp8 == nullptr;
  a.rope_dims = L.rope_dims;
  a.out = L.out;
  a.lse = L.lse;
  a.rope = make_rope_table(L.rope_base, L.rope_dims);
  a.units = p.splits * L.total_q;
  // 1-D grid with the head groups of one split on one XCD (wg_coords)
  const dim3 grid_xcd((unsigned)(8 * (int64_t)p.head_groups * ((a.units + 7) / 8)));
  switch (L.kv->dtype) {
    case CSA_FP8_E4M3: launch_q<CSA_FP8_E4M3>(a, L.q_dtype, dim, grid_xcd, stream); break;
    case CSA_BF16: launch_q<CSA_BF16>(a, L.q_dtype, dim, grid_xcd, stream); break;
    default: launch_q<CSA_F32>(a, L.q_dtype, dim, grid_xcd, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.direct) return e;
  MergeArgs m{};
  m.n_heads = L.n_heads;
  m.splits = p.splits;
  m.hgp = a.hgp;
  m.dim = dim;
  m.rope_dims = L.rope_dims;
  m.rope = a.rope;
  m.q_pos = L.q_pos;
  m.part_o = a.part_o;
  m.part_ml = a.part_ml;
  m.out = L.out;
  m.lse = L.lse;
  m.out_fp8 = L.out_fp8;
  m.out_scales = L.out_scales;
  hipLaunchKernelGGL(attn_merge, dim3((L.n_heads + 3) / 4, L.total_q), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace csa
