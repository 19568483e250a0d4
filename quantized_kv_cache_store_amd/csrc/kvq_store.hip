// Quantize-on-append store kernel and the query-preparation test export.
//
// [tract-RFC] Architecture > Data flow (decode), append step: rotate (fast
// Walsh-Hadamard), per-token symmetric int4, pack -- or keep the newest tokens
// as exact f32 rows (n_recent); the on-device append kernel is the piece the
// Metal integration section leaves unwritten.  [FreeToken-268] Storage layouts
// give the q4_0 / q6_0 block encodings (and its Summary the 8-bit q8_0 block
// at 1.0625 bytes per element); [Open-TQ-Metal] Background gives the
// per-group asymmetric int4.  Every stored value is a bit-exact function of
// the f32 inputs: IEEE f32 add/sub/mul/div, round-half-even to integers, fp16
// fields rounded to nearest even after clamping to +-65504.

#include "kvq_internal.h"

namespace kvq {

struct StoreArgs {
  const float* k_new;
  const float* v_new;
  const int32_t* slot;
  const int32_t* batch_idx;
  const int32_t* pos;
  const int32_t* seq_len;
  uint8_t* payload[2];
  uint8_t* record[2];
  float* ring[2];
  int n_rows;      // n_tok * Hkv * 2
  int Hkv;
  int page_shift;  // log2(page_size)
  int n_recent;
  // chunk form (bt set): token tok = b * n_q + i goes to position q_start[b] + i of row b, its slot
  // read from the block table; the row's length after the append is q_start[b] + n_q
  const int32_t* bt;
  const int32_t* q_start;
  int max_pages, n_q;
  // rotation only (rot set, Hadamard layout): the rotated f32 rows go to rot[kv] [n_tok][Hkv][D] and
  // nothing is stored in the cache
  float* rot[2];
};

__device__ __forceinline__ uint32_t pack8(const int* n) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) w |= (uint32_t)(n[e] & 0xF) << (4 * e);
  return w;
}

__device__ __forceinline__ uint32_t top8(const int* n) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) w |= (uint32_t)((n[e] >> 4) & 0x3) << (2 * e);
  return w;
}

__device__ __forceinline__ uint16_t f16_bits_sat(float x) {
  x = fminf(fmaxf(x, -65504.0f), 65504.0f);
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float f16_round_sat(float x) {
  x = fminf(fmaxf(x, -65504.0f), 65504.0f);
  return (float)(_Float16)x;
}

// One 16-lane row group encodes one row (token, kv head, K or V); four per wave.
template <int L, int D>
__global__ __launch_bounds__(256) void store_kernel(StoreArgs a) {
#pragma clang fp contract(off)
  using T = Layout<L, D>;
  constexpr int E = D / 16;              // elements per lane
  constexpr int LPG = 32 / E;            // lanes per 32-element group
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15;
  const int row = (blockIdx.x * 256 + threadIdx.x) >> 4;
  const bool active = row < a.n_rows;
  const int r = active ? row : 0;
  const int kv = r & 1;
  const int h = (r >> 1) % a.Hkv;
  const int tok = (r >> 1) / a.Hkv;

  float x[E];
  const float* src = (kv ? a.v_new : a.k_new) + ((size_t)tok * a.Hkv + h) * D + sub * E;
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const float4 v = active ? *reinterpret_cast<const float4*>(src + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
  }

  if (L == HAD) {
    // in-lane stages h < E
#pragma unroll
    for (int hh = 1; hh < E; hh <<= 1) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if ((i & hh) == 0) {
          const float p = x[i], q = x[i + hh];
          x[i] = p + q;
          x[i + hh] = p - q;
        }
      }
    }
    // cross-lane stages h = E .. D/2: partner lane differs in bit h/E of sub
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const bool upper = (sub & m) != 0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float y = __shfl_xor(x[i], m);
        x[i] = upper ? (y - x[i]) : (x[i] + y);
      }
    }
    const float c = hadamard_norm<D>();
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = x[i] * c;
    if (a.rot[0]) {
      if (active) {
        float* dst = a.rot[kv] + ((size_t)tok * a.Hkv + h) * D + sub * E;
#pragma unroll
        for (int e = 0; e < E; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
      }
      return;
    }
  }

  int s = 0, b = 0, p = 0, len = 0;   // slot; batch row, position and row length (window only)
  bool ok = active;
  if (a.bt) {
    b = tok / a.n_q;
    p = active ? a.q_start[b] + (tok - b * a.n_q) : 0;
    const int pg = p >> a.page_shift;
    ok = ok && p >= 0 && pg < a.max_pages;          // positions the block table does not cover are skipped
    s = ok ? (a.bt[(size_t)b * a.max_pages + pg] << a.page_shift) | (p & ((1 << a.page_shift) - 1)) : 0;
    len = active ? a.q_start[b] + a.n_q : 0;
  } else {
    s = active ? a.slot[tok] : 0;
    if (a.n_recent > 0 && active) {
      b = a.batch_idx[tok];
      p = a.pos[tok];
      len = a.seq_len[b];
    }
  }
  const size_t prow = ((size_t)(s >> a.page_shift) * a.Hkv + h) * ((size_t)1 << a.page_shift) +
                      (size_t)(s & ((1 << a.page_shift) - 1));

  // recent window: exact f32 row (rotated for HAD) at ring slot pos % n_recent
  if (a.n_recent > 0 && ok) {
    if (p >= len - a.n_recent) {
      float* dst = a.ring[kv] + (((size_t)b * a.Hkv + h) * a.n_recent + (p % a.n_recent)) * D + sub * E;
#pragma unroll
      for (int e = 0; e < E; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
    }
  }

  int n[E];
  uint8_t* rec = a.record[kv] + prow * T::SB;
  if (L == HAD) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(x[i]));
    m = wave_max16(m);
    const float sc = m / 8.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) n[i] = sc == 0.0f ? 0 : (int)fminf(fmaxf(rintf(x[i] / sc), -8.0f), 7.0f);
    if (ok && sub == 0) *reinterpret_cast<float*>(rec) = sc;
  } else if (L == Q40 || L == Q60 || L == Q80) {
    constexpr float M = (L == Q40) ? 8.0f : (L == Q60 ? 32.0f : 128.0f);
    constexpr float lo = -M, hi = M - 1.0f;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
    for (int o = 1; o < LPG; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float d32 = m / M;
    const float d = f16_round_sat(d32);
#pragma unroll
    for (int i = 0; i < E; ++i) n[i] = d == 0.0f ? 0 : (int)fminf(fmaxf(rintf(x[i] / d), lo), hi);
    if (ok && (sub % LPG) == 0) reinterpret_cast<uint16_t*>(rec)[sub / LPG] = f16_bits_sat(d32);
  } else {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < E; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
#pragma unroll
    for (int o = 1; o < LPG; o <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, o));
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    const float range = mx - mn;
    const float s32 = range / 15.0f;
    const float sc = f16_round_sat(s32);
    const float z = f16_round_sat(mn);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float t = x[i] - z;
      n[i] = sc == 0.0f ? 0 : (int)fminf(fmaxf(rintf(t / sc), 0.0f), 15.0f);
    }
    if (ok && (sub % LPG) == 0)
      reinterpret_cast<uint32_t*>(rec)[sub / LPG] = (uint32_t)f16_bits_sat(s32) | ((uint32_t)f16_bits_sat(mn) << 16);
  }

  // Payload words are gathered so that each write is 16 bytes: the lane's packed words, and those of
  // the next lanes of its row (DPP row shifts, within the 16 lanes of the row), go out from every
  // 16 / (bytes per lane)-th lane.  Every lane of a row takes part in the shifts (ok is row-uniform).
  uint8_t* pay = a.payload[kv] + prow * T::PB;
  auto from = [](uint32_t w, auto dn) {   // the word of lane sub + n of this row (n = 1, 2, 3)
    constexpr int n = decltype(dn)::value;
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x100 + n, 0xF, 0xF, false);   // row_shl:n
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if (L == Q80) {
    // one two's-complement byte per code, element order: the lane's E codes at byte sub * E
    uint32_t w[E / 4];
#pragma unroll
    for (int i = 0; i < E / 4; ++i)
      w[i] = (uint32_t)(n[4 * i] & 0xFF) | ((uint32_t)(n[4 * i + 1] & 0xFF) << 8) |
             ((uint32_t)(n[4 * i + 2] & 0xFF) << 16) | ((uint32_t)(n[4 * i + 3] & 0xFF) << 24);
    if constexpr (E == 8) {   // 8 bytes per lane: lane pairs
      const uint32_t w2 = from(w[0], I1{}), w3 = from(w[1], I1{});
      if (ok && (sub & 1) == 0) reinterpret_cast<uint4*>(pay)[sub >> 1] = make_uint4(w[0], w[1], w2, w3);
    } else {
      if (ok) reinterpret_cast<uint4*>(pay)[sub] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else if (L != Q60) {
    if (E == 8) {   // 4 bytes per lane: lane quads
      const uint32_t w0 = pack8(n);
      const uint32_t w1 = from(w0, I1{}), w2 = from(w0, I2{}), w3 = from(w0, I3{});
      if (ok && (sub & 3) == 0) reinterpret_cast<uint4*>(pay)[sub >> 2] = make_uint4(w0, w1, w2, w3);
    } else {        // 8 bytes per lane: lane pairs
      const uint32_t w0 = pack8(n), w1 = pack8(n + 8);
      const uint32_t w2 = from(w0, I1{}), w3 = from(w1, I1{});
      if (ok && (sub & 1) == 0) reinterpret_cast<uint4*>(pay)[sub >> 1] = make_uint4(w0, w1, w2, w3);
    }
  } else {
    if (!ok) return;
    // q6_0: 24-byte blocks (16 bytes of low nibbles, then 8 of top-bit pairs), not 16-byte aligned
    // lane holds octets o = sub*E/8 .. ; octet o lives in block o/4 at slot o%4
    if (E == 8) {
      const int g = sub >> 2, c = sub & 3;
      *reinterpret_cast<uint32_t*>(pay + 24 * g + 4 * c) = pack8(n);
      *reinterpret_cast<uint16_t*>(pay + 24 * g + 16 + 2 * c) = (uint16_t)top8(n);
    } else {
      const int g = sub >> 1, c = (sub & 1) * 2;
      *reinterpret_cast<uint2*>(pay + 24 * g + 4 * c) = make_uint2(pack8(n), pack8(n + 8));
      *reinterpret_cast<uint32_t*>(pay + 24 * g + 16 + 2 * c) = top8(n) | (top8(n + 8) << 16);
    }
  }
}

// Query preparation export: 16 vectors per block.
template <int L, int D>
__global__ __launch_bounds__(256) void quantize_q_kernel(const float* q, int n_vec, int8_t* q8, float* sq) {
  __shared__ __align__(16) float qf[16 * D];
  __shared__ __align__(16) int8_t q8s[16 * D];
  __shared__ float sqs[16];
  __shared__ int qsum[16 * (D / 32)];
  const int v0 = blockIdx.x * 16;
  for (int idx = threadIdx.x; idx < 16 * D; idx += 256) {
    const int v = v0 + idx / D;
    qf[idx] = v < n_vec ? q[(size_t)v * D + idx % D] : 0.0f;
  }
  __syncthreads();
  prepare_query_lds<L, D>(qf, q8s, sqs, qsum);
  for (int idx = threadIdx.x; idx < 16 * D; idx += 256) {
    const int v = v0 + idx / D;
    if (v < n_vec) q8[(size_t)v * D + idx % D] = q8s[idx];
  }
  if (threadIdx.x < 16 && v0 + (int)threadIdx.x < n_vec) sq[v0 + threadIdx.x] = sqs[threadIdx.x];
}

template <int L, int D>
static void launch_store(const StoreArgs& a, hipStream_t st) {
  const int blocks = (a.n_rows + 15) / 16;
  hipLaunchKernelGGL((store_kernel<L, D>), dim3(blocks), dim3(256), 0, st, a);
}

typedef void (*store_fn)(const StoreArgs&, hipStream_t);

static store_fn pick_store(int layout, int D) {
  const int di = D == 256 ? 1 : 0;
  static const store_fn tab[kNumLayouts][2] = {
      {launch_store<HAD, 128>, launch_store<HAD, 256>},
      {launch_store<Q40, 128>, launch_store<Q40, 256>},
      {launch_store<Q60, 128>, launch_store<Q60, 256>},
      {launch_store<ASYM, 128>, launch_store<ASYM, 256>},
      {launch_store<Q80, 128>, launch_store<Q80, 256>},
  };
  return tab[layout][di];
}

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_store(const kvq_cache* c, const float* k_new, const float* v_new, int32_t n_tok,
                                const int32_t* slot, const int32_t* batch_idx, const int32_t* pos,
                                const int32_t* seq_len, void* stream) {
  kvq_status st = validate_cache(c);
  if (st != KVQ_OK) return st;
  if (n_tok < 0) return fail(KVQ_ERR_INVALID_ARG, "n_tok must be >= 0");
  if (n_tok == 0) return KVQ_OK;
  if (!k_new || !v_new || !slot) return fail(KVQ_ERR_INVALID_ARG, "k_new, v_new and slot must be non-null");
  if (c->n_recent > 0 && (!batch_idx || !pos || !seq_len))
    return fail(KVQ_ERR_INVALID_ARG, "batch_idx, pos and seq_len are required when n_recent > 0");
  if ((size_t)n_tok * c->num_kv_heads * 2 > (size_t)INT32_MAX)
    return fail(KVQ_ERR_INVALID_ARG, "too many rows in one store");
  StoreArgs a;
  memset(&a, 0, sizeof(a));
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot = slot;
  a.batch_idx = batch_idx;
  a.pos = pos;
  a.seq_len = seq_len;
  a.payload[0] = (uint8_t*)c->k_payload;
  a.payload[1] = (uint8_t*)c->v_payload;
  a.record[0] = (uint8_t*)c->k_scale;
  a.record[1] = (uint8_t*)c->v_scale;
  a.ring[0] = c->k_recent;
  a.ring[1] = c->v_recent;
  a.n_rows = n_tok * c->num_kv_heads * 2;
  a.Hkv = c->num_kv_heads;
  a.page_shift = __builtin_ctz((unsigned)c->page_size);
  a.n_recent = c->n_recent;
  pick_store(c->layout, c->head_dim)(a, (hipStream_t)stream);
  return check_launch("store kernel");
}

namespace kvq {
// The Hadamard-rotated f32 rows of n_tok tokens of k_new, v_new [n_tok][Hkv][D] into kr, vr (same
// shape), by the store kernel's own rotation; nothing is stored.  For the full-precision prefill.
kvq_status launch_rotate_rows(const kvq_cache* c, const float* k_new, const float* v_new, int n_tok, float* kr,
                              float* vr, hipStream_t st) {
  StoreArgs a;
  memset(&a, 0, sizeof(a));
  a.k_new = k_new;
  a.v_new = v_new;
  a.n_rows = n_tok * c->num_kv_heads * 2;
  a.Hkv = c->num_kv_heads;
  a.page_shift = __builtin_ctz((unsigned)c->page_size);
  a.rot[0] = kr;
  a.rot[1] = vr;
  if (a.n_rows == 0) return KVQ_OK;
  (c->head_dim == 256 ? launch_store<HAD, 256> : launch_store<HAD, 128>)(a, st);
  return check_launch("rotation kernel");
}
}  // namespace kvq

extern "C" kvq_status kvq_store_chunk(const kvq_cache* c, const float* k_new, const float* v_new, int32_t batch,
                                      int32_t n_q, const int32_t* q_start, const int32_t* block_table,
                                      int32_t max_pages, int32_t max_seq_len, void* stream) {
  kvq_status st = validate_cache(c);
  if (st != KVQ_OK) return st;
  if (batch < 1 || n_q < 0) return fail(KVQ_ERR_INVALID_ARG, "batch must be >= 1 and n_q >= 0");
  if (n_q == 0) return KVQ_OK;
  if (!k_new || !v_new || !q_start || !block_table)
    return fail(KVQ_ERR_INVALID_ARG, "k_new, v_new, q_start and block_table must be non-null");
  if (max_seq_len < n_q || max_pages < 1 || (int64_t)max_pages * c->page_size < max_seq_len)
    return fail(KVQ_ERR_INVALID_ARG, "max_pages_per_seq * page_size must cover max_seq_len >= n_q");
  if (c->n_recent > 0 && batch > c->max_batch) return fail(KVQ_ERR_INVALID_ARG, "batch above the window rings' max_batch");
  if ((int64_t)batch * n_q * c->num_kv_heads * 2 > (int64_t)INT32_MAX)
    return fail(KVQ_ERR_INVALID_ARG, "too many rows in one store");
  StoreArgs a;
  memset(&a, 0, sizeof(a));
  a.k_new = k_new;
  a.v_new = v_new;
  a.payload[0] = (uint8_t*)c->k_payload;
  a.payload[1] = (uint8_t*)c->v_payload;
  a.record[0] = (uint8_t*)c->k_scale;
  a.record[1] = (uint8_t*)c->v_scale;
  a.ring[0] = c->k_recent;
  a.ring[1] = c->v_recent;
  a.n_rows = batch * n_q * c->num_kv_heads * 2;
  a.Hkv = c->num_kv_heads;
  a.page_shift = __builtin_ctz((unsigned)c->page_size);
  a.n_recent = c->n_recent;
  a.bt = block_table;
  a.q_start = q_start;
  a.max_pages = max_pages;
  a.n_q = n_q;
  pick_store(c->layout, c->head_dim)(a, (hipStream_t)stream);
  return check_launch("store kernel");
}

extern "C" kvq_status kvq_debug_quantize_q(int32_t layout, const float* q, int32_t n_vec, int32_t head_dim,
                                           int8_t* q8, float* sq, void* stream) {
  if (payload_bytes_rt(layout, head_dim) == 0)
    return fail(KVQ_ERR_UNSUPPORTED, "layout %d with head_dim %d is not supported", layout, head_dim);
  if (n_vec < 0) return fail(KVQ_ERR_INVALID_ARG, "n_vec must be >= 0");
  if (n_vec == 0) return KVQ_OK;
  if (!q || !q8 || !sq) return fail(KVQ_ERR_INVALID_ARG, "q, q8 and sq must be non-null");
  const dim3 grid((n_vec + 15) / 16);
  hipStream_t st = (hipStream_t)stream;
  const bool had = layout == HAD;
  if (head_dim == 128) {
    if (had) hipLaunchKernelGGL((quantize_q_kernel<HAD, 128>), grid, dim3(256), 0, st, q, n_vec, q8, sq);
    else hipLaunchKernelGGL((quantize_q_kernel<Q40, 128>), grid, dim3(256), 0, st, q, n_vec, q8, sq);
  } else {
    if (had) hipLaunchKernelGGL((quantize_q_kernel<HAD, 256>), grid, dim3(256), 0, st, q, n_vec, q8, sq);
    else hipLaunchKernelGGL((quantize_q_kernel<Q40, 256>), grid, dim3(256), 0, st, q, n_vec, q8, sq);
  }
  return check_launch("query preparation kernel");
}
