// Pieces shared by the decode and prefill attention kernels: the argument block,
// row geometry, f32 window partial, and host-side argument handling.
#pragma once

#include "kvq_internal.h"

namespace kvq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define KVQ_LOG2E 1.4426950408889634f

struct AttendArgs {
  const uint8_t* kp;
  const uint8_t* vp;
  const uint8_t* ks;
  const uint8_t* vs;
  const float* kring;
  const float* vring;
  const float* q;
  float* ws;
  const int32_t* block_table;
  const int32_t* seq_len;
  const int32_t* q_start;   // [batch] position of query 0 (causal prefill), else null
  const float* qrot;        // prepared rows (prefill): f32 query, rotated for HAD, [rows][D], else null
  const int8_t* q8p;        // prepared rows: int8 query [rows][D]
  const float* sqp;         // prepared rows: its scale [rows]
  const int* qsump;         // prepared rows: sum of q8 per 32-element block [rows][D / 32]
  int32_t* dbg;
  int Hkv, Hq, G, page_shift, n_recent, max_pages, chunk, nc1, max_seq_len;
  int n_q;       // queries per batch row (1 for decode)
  int batch;     // batch rows (decode: the grid is one-dimensional)
  int ngroups;   // blocks per row tile along the sequence: chunk groups of four, + 1 for the window
  int cpw;       // consecutive chunks each wave of the decode kernel streams (1 elsewhere)
  int causal;    // rows see t <= q_start + i
  int skip;      // causal skip: stop streaming past the tile's last visible token
  float alpha;
};

// Row R of (b, hk) is query i = R / G of head hk * G + R % G; its flat index in
// [batch][n_q][Hq] addresses q, out and (times the chunk count) the partials.
__device__ __forceinline__ size_t row_index(const AttendArgs& a, int b, int hk, int R) {
  const int i = R / a.G;
  return ((size_t)b * a.n_q + i) * a.Hq + hk * a.G + (R - i * a.G);
}

// Last visible position of row R (rows past the tile's valid count see nothing).
__device__ __forceinline__ int row_limit(const AttendArgs& a, int qs0, int R, int nrows) {
  if (R >= nrows) return -1;
  return a.causal ? qs0 + R / a.G : 0x7fffffff;
}

template <int D>
__host__ __device__ constexpr int prologue_lds_bytes() {
  return 16 * D * 4 + 16 * D + 16 * 4 + 16 * (D / 32) * 4;
}

// Reductions over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48), on the VALU:
// v_permlane16_swap / v_permlane32_swap applied to two copies of a value leave in the two
// registers the value of the lane and of its partner row, in row order, so both lanes of a pair
// compute the same result.  Written as inline assembly with both registers read-write (the
// compiler's built-in for it folds its two results into one), with the wait states the swap
// needs after the VALU writes of its operands.
__device__ __forceinline__ void row_pair(float v, int swap32, float& lo, float& hi) {
  float x = v, y = v;
  if (swap32)
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  else
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  lo = x;
  hi = y;
}

__device__ __forceinline__ float max_over_rows(float v) {
  float a, b;
  row_pair(v, 0, a, b);
  row_pair(fmaxf(a, b), 1, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float sum_over_rows(float v) {
  float a, b;
  row_pair(v, 0, a, b);
  row_pair(a + b, 1, a, b);
  return a + b;
}

__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// q6_0 octet (low-nibble dword + 16 bits of top-bit pairs) -> biased 6-bit codes
// (code + 32) as bytes, even elements [0,2,4,6] in `ev`, odd [1,3,5,7] in `od`.
__device__ __forceinline__ void q6_octet(uint32_t lo, uint32_t hi16, uint32_t& ev, uint32_t& od) {
  const uint32_t w = __builtin_amdgcn_perm(hi16, hi16, 0x01010000u);   // bytes [b0, b0, b1, b1]
  const uint32_t te = ((w << 4) & 0x00300030u) | (w & 0x30003000u);
  const uint32_t to = ((w << 2) & 0x00300030u) | ((w >> 2) & 0x30003000u);
  ev = ((lo & 0x0F0F0F0Fu) | te) ^ 0x20202020u;
  od = (((lo >> 4) & 0x0F0F0F0Fu) | to) ^ 0x20202020u;
}

// Window partial: exact f32 rows of the newest tokens (HAD: rotated basis), for the rows
// row0 .. row0 + nvalid - 1 of (b, hk), each masked by its limit.  The window is walked in
// tiles of 16 tokens staged in LDS with an online softmax: thread (row = tid / 16, j = tid % 16)
// scores token j of the tile for its row and accumulates output elements d = j + 16 e.
// LDS: the query preparation area, then K tile [16][D + 4] (padded rows: conflict-free float4
// reads), V tile [16][D], P tile [16][16].
template <int D>
__host__ __device__ constexpr int window_lds_bytes() {
  return prologue_lds_bytes<D>() + 16 * (D + 4) * 4 + 16 * D * 4 + 16 * 16 * 4;
}

template <int L, int D>
__device__ __forceinline__ void window_partial(const AttendArgs& a, unsigned char* smem, int b, int hk, int S, int row0,
                                               int nvalid, int qs0) {
  constexpr int E = D / 16;
  constexpr int KST = D + 4;
  constexpr int NL = D / 64;          // float4 of one tile's K (and of its V) per thread
  float* qf = reinterpret_cast<float*>(smem);
  int8_t* q8 = reinterpret_cast<int8_t*>(qf + 16 * D);
  float* sq = reinterpret_cast<float*>(q8 + 16 * D);
  int* qsum = reinterpret_cast<int*>(sq + 16);
  float* kt = reinterpret_cast<float*>(smem + prologue_lds_bytes<D>());
  float* vt = kt + 16 * KST;
  float* pt = vt + 16 * D;
  const int tid = threadIdx.x;
  const int nrows = a.n_q * a.G;
  const float* qsrc = a.qrot ? a.qrot : a.q;     // prepared rows are already rotated
  for (int idx = tid; idx < 16 * D; idx += 256) {
    const int row = idx / D;
    qf[idx] = row < nvalid ? qsrc[row_index(a, b, hk, row0 + row) * D + idx % D] : 0.0f;
  }
  __syncthreads();
  if (!a.qrot) prepare_query_lds<L, D>(qf, q8, sq, qsum);
  const int W = min(S, a.n_recent);
  const int w0 = S - W;
  const size_t ring0 = ((size_t)b * a.Hkv + hk) * a.n_recent;
  const float cl = a.alpha * KVQ_LOG2E;
  const int row = tid >> 4, j = tid & 15;
  const int lim = row < nvalid ? row_limit(a, qs0, row0 + row, nrows) : -1;
  float m = -INFINITY, l = 0.0f;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.0f;
  // tile loads in registers, one tile ahead (rows past the window: zeros)
  float4 kreg[NL], vreg[NL];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int idx = tid + 256 * n;
      const int tt = idx / (D / 4), c4 = idx % (D / 4);
      kreg[n] = make_float4(0.f, 0.f, 0.f, 0.f);
      vreg[n] = kreg[n];
      if (t0 + tt < W) {
        int slot = w0 + t0 + tt;
        slot -= (slot / a.n_recent) * a.n_recent;
        const size_t ro = (ring0 + (size_t)slot) * D + 4 * c4;
        kreg[n] = *reinterpret_cast<const float4*>(a.kring + ro);
        vreg[n] = *reinterpret_cast<const float4*>(a.vring + ro);
      }
    }
  };
  if (W > 0) load_tile(0);
  for (int t0 = 0; t0 < W; t0 += 16) {
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int idx = tid + 256 * n;
      const int tt = idx / (D / 4), c4 = idx % (D / 4);
      *reinterpret_cast<float4*>(kt + tt * KST + 4 * c4) = kreg[n];
      *reinterpret_cast<float4*>(vt + tt * D + 4 * c4) = vreg[n];
    }
    __syncthreads();
    if (t0 + 16 < W) load_tile(t0 + 16);
    // score of token t0 + j for this thread's row
    float acc = 0.0f;
    const float* qr = qf + row * D;
    const float* kr = kt + j * KST;
#pragma unroll 8
    for (int d = 0; d < D; d += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(kr + d);
      const float4 q4 = *reinterpret_cast<const float4*>(qr + d);
      acc += q4.x * k4.x + q4.y * k4.y + q4.z * k4.z + q4.w * k4.w;
    }
    const int t = t0 + j;
    const float x = (t < W && w0 + t <= lim) ? acc * cl : -INFINITY;
    float tmax = x;
#pragma unroll
    for (int k = 1; k < 16; k <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, k));
    const float m_new = fmaxf(m, tmax);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // a row that sees nothing yet: p = 0
    const float corr = exp2f(m - m_use);
    const float p = exp2f(x - m_use);
    float ps = p;
#pragma unroll
    for (int k = 1; k < 16; k <<= 1) ps += __shfl_xor(ps, k);
    l = l * corr + ps;
    m = m_new;
    pt[row * 16 + j] = p;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float acc_o = o[e] * corr;
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) acc_o += pt[row * 16 + tt] * vt[tt * D + j + 16 * e];
      o[e] = acc_o;
    }
    __syncthreads();
  }
  if (row < nvalid) {
    float* dst = a.ws + (row_index(a, b, hk, row0 + row) * a.nc1 + (a.nc1 - 1)) * partial_stride(D);
#pragma unroll
    for (int e = 0; e < E; ++e) dst[j + 16 * e] = o[e];
    if (j == 0) {
      dst[D] = m;
      dst[D + 1] = l;
    }
  }
}

// ----------------------------------------------------------------------------- host side

static inline int chunks_of(int max_seq_len, int chunk) { return (max_seq_len + chunk - 1) / chunk; }

static inline kvq_status check_attend_args(const kvq_cache* c, const void* q, int32_t batch, int32_t Hq,
                                           const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                                           int32_t max_seq_len) {
  kvq_status st = validate_cache(c);
  if (st != KVQ_OK) return st;
  if (!q || !block_table || !seq_len) return fail(KVQ_ERR_INVALID_ARG, "q, block_table and seq_len must be non-null");
  if (batch < 1) return fail(KVQ_ERR_INVALID_ARG, "batch must be >= 1");
  if (Hq < 1 || Hq % c->num_kv_heads) return fail(KVQ_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (max_pages < 1 || (int64_t)max_pages * c->page_size < max_seq_len)
    return fail(KVQ_ERR_INVALID_ARG, "max_pages_per_seq * page_size must cover max_seq_len");
  if (c->n_recent > 512) return fail(KVQ_ERR_UNSUPPORTED, "n_recent above 512");
  return KVQ_OK;
}

// Argument block for a launch over rows of n_q queries; ngroups is set for the decode kernel
// (chunk groups of four, + 1 window group) and replaced by the prefill.
static inline AttendArgs make_args(const kvq_cache* c, const float* q, int32_t Hq, int32_t n_q, float alpha,
                                   const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                                   int32_t max_seq_len, int32_t chunk, void* workspace) {
  AttendArgs a;
  memset(&a, 0, sizeof(a));
  a.kp = (const uint8_t*)c->k_payload;
  a.vp = (const uint8_t*)c->v_payload;
  a.ks = (const uint8_t*)c->k_scale;
  a.vs = (const uint8_t*)c->v_scale;
  a.kring = c->k_recent;
  a.vring = c->v_recent;
  a.q = q;
  a.ws = (float*)workspace;
  a.block_table = block_table;
  a.seq_len = seq_len;
  a.Hkv = c->num_kv_heads;
  a.Hq = Hq;
  a.G = Hq / c->num_kv_heads;
  a.page_shift = __builtin_ctz((unsigned)c->page_size);
  a.n_recent = c->n_recent;
  a.max_pages = max_pages;
  a.chunk = chunk;
  const int nch = chunks_of(max_seq_len, chunk);
  a.nc1 = nch + 1;
  a.max_seq_len = max_seq_len;
  a.n_q = n_q;
  a.ngroups = (nch + 3) / 4 + (c->n_recent > 0 ? 1 : 0);
  a.cpw = 1;
  a.alpha = alpha;
  return a;
}

// Blocks along x of the decode kernel: row tiles of tr rows times chunk groups (0 when there is
// nothing to do).
static inline int64_t grid_x(const AttendArgs& a, int tr) {
  const int64_t tiles = ((int64_t)a.n_q * a.G + tr - 1) / tr;
  return tiles * a.ngroups;
}

static inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Prepared query rows in a workspace, after the partials: [rotated f32 query rows x D] [int8
// query rows x D] [scale f32 rows] [block sums int32 rows x D / 32], each part 16-byte aligned.
struct RowPrep {
  size_t qrot, q8, sq, qsum, end;
};

static inline RowPrep row_prep_layout(size_t at, size_t rows, int D) {
  RowPrep w;
  w.qrot = align16(at);
  w.q8 = w.qrot + align16(rows * D * sizeof(float));
  w.sq = w.q8 + align16(rows * D);
  w.qsum = w.sq + align16(rows * sizeof(float));
  w.end = w.qsum + align16(rows * (D / 32) * sizeof(int));
  return w;
}

// Query preparation of n_vec rows of q (kvq_prefill.hip): int8 query, scale, block sums, and for
// the Hadamard layout the rotated f32 query.  Points a's prepared-row fields at them.
kvq_status launch_prepare_rows(const kvq_cache* c, const float* q, int n_vec, unsigned char* ws, const RowPrep& w,
                               AttendArgs& a, hipStream_t s);

// The online-softmax reduce over the partials of batch * rows_per_b rows (kvq_attend.hip).
kvq_status launch_reduce(const kvq_cache* c, float* out, int32_t batch, int32_t rows_per_b, const int32_t* seq_len,
                         int nc1, int32_t chunk, const float* ws, hipStream_t s);

}  // namespace kvq
