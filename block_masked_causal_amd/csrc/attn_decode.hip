// Block-decode attention for gfx950.
//
// In MARS inference each sequence appends B [MASK] queries and scores them in
// one forward; the queries read a block-level prefix KV cache and attend
// causally to each other (gist.science explainer on "MARS: Enabling
// Autoregressive Models Multi-Token Generation", sections 2C-2D;
// papernotes.org notes, key designs 3-4 / 关键设计 3-4).
//
// Design: the g = Hq/Hkv query heads of one KV head and the B rows of a
// sequence share every K/V element, so they are packed into 32-row query
// tiles (packed row j = r*g + head_in_group) and multiplied on MFMA. The work
// is HBM-bound (about 28 flop per byte at d = 128), so each K/V byte is read
// exactly once, straight from HBM into MFMA operands:
//   * S^T = K Q^T: lane (key i, half hf) reads 16 bytes of its key's row.
//   * O^T = V^T P^T: the V pages are stored transposed ([d][slot]), so the A
//     operand of lane (dim, hf) is two 8-byte reads of consecutive slots.
// The cache of one sequence is cut into chunks of kChunk keys (split-K); each
// workgroup handles one (chunk, KV head, sequence) and writes an unnormalised
// partial (O, running max, running sum); a merge kernel combines the chunks.
// Chunk 0 also handles the B new rows (causal among themselves).
#include "mars_common.hpp"

using namespace mars;

namespace {

constexpr int kChunk = 256;  // cache keys per split-K chunk (multiple of 32)
constexpr int kMaxQT = 4;    // at most 4 query tiles of 32 packed rows

struct DecodeArgs {
  const bf16_t* q;
  const bf16_t* k_new;
  const bf16_t* v_new;
  const bf16_t* k_cache;
  const bf16_t* v_cache;
  const int32_t* block_table;
  const int32_t* cache_len;
  bf16_t* o;
  float* part_o;   // [S][Hkv][nsplit][nrows_pad][D]
  float* part_ml;  // [S][Hkv][nsplit][nrows_pad][2]
  int32_t* status;
  int S, B, Hq, Hkv, group, page_size, max_pages, num_pages, nsplit, nrows_pad;
  float scale_log2;
};

template <int D>
__global__ __launch_bounds__(64 * kMaxQT) void decode_split_kernel(DecodeArgs p) {
  const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63, wq = threadIdx.x >> 6;
  const int j = lane & 31, hf = lane >> 5;
  const int nrows = p.group * p.B;
  if (wq * 32 >= nrows) return;  // wave-uniform: no barriers in this kernel

  int len = p.cache_len[s];
  const int cap = p.max_pages * p.page_size;
  if (len > cap) {
    if (split == 0 && kvh == 0 && threadIdx.x == 0) status_or(p.status, MARS_STATUS_CACHE_OVERFLOW);
    len = cap;
  }
  if (len < 0) len = 0;
  const int k_lo = split * kChunk;
  if (split > 0 && k_lo >= len) return;
  const int k_hi = min(len, k_lo + kChunk);

  // Packed query row of this lane: j' = r * g + head_in_group.
  const int qi = wq * 32 + j;
  const bool qvalid = qi < nrows;
  const int qr = qvalid ? qi / p.group : 0;
  const int qh = kvh * p.group + (qvalid ? qi % p.group : 0);
  bf16x8 qf[D / 16];
  {
    const bf16_t* qrow = p.q + (((size_t)s * p.B + qr) * p.Hq + qh) * D + 8 * hf;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qf[c] = qvalid ? *(const bf16x8*)(qrow + 16 * c) : bf16x8{};
  }

  const int32_t* table = p.block_table + (size_t)s * p.max_pages;
  const size_t kpage = (size_t)p.Hkv * p.page_size * D;  // elements per page (all heads)
  const bf16_t* kbase = p.k_cache + (size_t)kvh * p.page_size * D;
  const bf16_t* vbase = p.v_cache + (size_t)kvh * D * p.page_size;

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;
  bool bad_page = false;

  auto page_of = [&](int pos, bool& ok) -> int {
    const int pg = table[pos / p.page_size];
    ok = (pg >= 0) & (pg < p.num_pages);
    bad_page |= !ok;
    return ok ? pg : 0;
  };

  // One 32-key step: S^T, online softmax, O^T update. `kmask(c)` says whether
  // key slot c (0..31 within the step) is live for this lane's query.
  auto step = [&](const bf16x8 (&ka)[D / 16], const bf16x8 (&va)[D / 32][2], auto live) {
    f32x16 sc = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) sc = mfma32(ka[c], qf[c], sc);
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 8 * (r >> 2) + 4 * hf + (r & 3);
      const float x = live(c) ? sc[r] * p.scale_log2 : -INFINITY;
      sc[r] = x;
      mt = fmaxf(mt, x);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt);
    const float mb = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - mb);
    float rsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(sc[r] - mb);
      sc[r] = e;
      rsum += e;
    }
    l = l * alpha + rsum;
    m = mnew;
    bf16x8 pb[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[kc][e] = (bf16_t)sc[8 * kc + e];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      o[i] *= alpha;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) o[i] = mfma32(va[i][kc], pb[kc], o[i]);
    }
  };

  // ---- cached prefix keys [k_lo, k_hi) -------------------------------------
  for (int c0 = k_lo; c0 < k_hi; c0 += 32) {
    bf16x8 ka[D / 16];
    {
      const int pos = c0 + j;
      bool ok = false;
      const int pg = pos < k_hi ? page_of(pos, ok) : 0;
      const bf16_t* kr = kbase + pg * kpage + (size_t)(pos % p.page_size) * D + 8 * hf;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) ka[c] = ok ? *(const bf16x8*)(kr + 16 * c) : bf16x8{};
    }
    bf16x8 va[D / 32][2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      // keys 16kc + 4hf + {0..3} and 16kc + 8 + 4hf + {0..3} of this step
      const int p0 = c0 + 16 * kc + 4 * hf;
      const int p1 = p0 + 8;
      bool ok0 = false, ok1 = false;
      const int pg0 = p0 < k_hi ? page_of(p0, ok0) : 0;
      const int pg1 = p1 < k_hi ? page_of(p1, ok1) : 0;
      const int n0 = min(4, k_hi - p0), n1 = min(4, k_hi - p1);  // live keys in each group
      const bf16_t* v0 = vbase + pg0 * kpage + (p0 % p.page_size);
      const bf16_t* v1 = vbase + pg1 * kpage + (p1 % p.page_size);
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const int d = 32 * i + j;
        u32x2 lo = ok0 ? *(const u32x2*)(v0 + (size_t)d * p.page_size) : u32x2{};
        u32x2 hi = ok1 ? *(const u32x2*)(v1 + (size_t)d * p.page_size) : u32x2{};
        // zero the slots past the end of the chunk (they may hold stale data)
        if (n0 < 4) {
          if (n0 <= 0) lo = u32x2{};
          else if (n0 == 1) { lo[0] &= 0xFFFFu; lo[1] = 0; }
          else if (n0 == 2) lo[1] = 0;
          else lo[1] &= 0xFFFFu;
        }
        if (n1 < 4) {
          if (n1 <= 0) hi = u32x2{};
          else if (n1 == 1) { hi[0] &= 0xFFFFu; hi[1] = 0; }
          else if (n1 == 2) hi[1] = 0;
          else hi[1] &= 0xFFFFu;
        }
        u32x4 packed = {lo[0], lo[1], hi[0], hi[1]};
        va[i][kc] = __builtin_bit_cast(bf16x8, packed);
      }
    }
    const int nlive = k_hi - c0;
    step(ka, va, [&](int c) { return c < nlive; });
  }

  // ---- the B new rows, causal among themselves (chunk 0 only) --------------
  if (split == 0) {
    bf16x8 ka[D / 16];
    {
      const bf16_t* kr = p.k_new + (((size_t)s * p.B + (j < p.B ? j : 0)) * p.Hkv + kvh) * D + 8 * hf;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) ka[c] = j < p.B ? *(const bf16x8*)(kr + 16 * c) : bf16x8{};
    }
    bf16x8 va[D / 32][2];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int d = 32 * i + j;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = 16 * kc + (e < 4 ? 4 * hf + e : 8 + 4 * hf + (e - 4));
          va[i][kc][e] = key < p.B ? p.v_new[(((size_t)s * p.B + key) * p.Hkv + kvh) * D + d]
                                   : (bf16_t)0.f;
        }
      }
    }
    step(ka, va, [&](int c) { return c <= qr && c < p.B; });
  }

  if (bad_page) status_or(p.status, MARS_STATUS_BAD_PAGE);

  // ---- partial result for this chunk ---------------------------------------
  const float lt = l + __shfl_xor(l, 32);
  if (!qvalid) return;
  const size_t prow = (((size_t)s * p.Hkv + kvh) * p.nsplit + split) * p.nrows_pad + qi;
  float* po = p.part_o + prow * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v4 = {o[i][4 * g], o[i][4 * g + 1], o[i][4 * g + 2], o[i][4 * g + 3]};
      *(f32x4*)(po + 32 * i + 8 * g + 4 * hf) = v4;
    }
  if (hf == 0) {
    p.part_ml[prow * 2 + 0] = m;
    p.part_ml[prow * 2 + 1] = lt;
  }
}

// One wave per (sequence, KV head, packed query row): combine the chunks.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs p) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nrows = p.group * p.B;
  const int total = p.S * p.Hkv * nrows;
  if (wave >= total) return;
  const int qi = wave % nrows;
  const int kvh = (wave / nrows) % p.Hkv;
  const int s = wave / (nrows * p.Hkv);
  int len = p.cache_len[s];
  len = min(max(len, 0), p.max_pages * p.page_size);
  const int nsp = max(1, (len + kChunk - 1) / kChunk);

  const size_t base = (((size_t)s * p.Hkv + kvh) * p.nsplit) * p.nrows_pad + qi;
  const size_t stride = p.nrows_pad;
  float M = -INFINITY;
  for (int sp = 0; sp < nsp; ++sp) M = fmaxf(M, p.part_ml[(base + sp * stride) * 2]);
  const float Mb = M == -INFINITY ? 0.f : M;
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float lsum = 0.f;
  for (int sp = 0; sp < nsp; ++sp) {
    const size_t row = base + sp * stride;
    const float w = fast_exp2(p.part_ml[row * 2] - Mb);
    lsum += w * p.part_ml[row * 2 + 1];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += w * p.part_o[row * D + lane * PER + e];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int r = qi / p.group, h = kvh * p.group + qi % p.group;
  bf16_t* orow = p.o + (((size_t)s * p.B + r) * p.Hq + h) * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[e] = (bf16_t)(acc[e] * inv);
}

size_t decode_ws_bytes(int S, int B, int Hq, int Hkv, int D, int page_size, int max_pages,
                       int* nsplit_out, int* nrows_pad_out) {
  const long long cap = (long long)max_pages * page_size;
  const int nsplit = (int)std::max<long long>(1, (cap + kChunk - 1) / kChunk);
  const int nrows = (Hq / Hkv) * B;
  const int nrows_pad = ((nrows + 31) / 32) * 32;
  if (nsplit_out) *nsplit_out = nsplit;
  if (nrows_pad_out) *nrows_pad_out = nrows_pad;
  const size_t rows = (size_t)S * Hkv * nsplit * nrows_pad;
  const size_t ob = rows * D * sizeof(float);
  const size_t ob_al = (ob + 255) & ~(size_t)255;
  return ob_al + rows * 2 * sizeof(float);
}

bool decode_sizes_ok(int S, int B, int Hq, int Hkv, int D, int page_size, int max_pages) {
  if (S < 1 || B < 1 || B > 32 || Hq < 1 || Hkv < 1 || Hq % Hkv) return false;
  if ((Hq / Hkv) * B > 32 * kMaxQT) return false;
  if (page_size < 16 || page_size % 16 || max_pages < 1) return false;
  if (S > 65535 || Hkv > 65535) return false;
  if ((long long)max_pages * page_size > (1LL << 30)) return false;
  (void)D;
  return true;
}

}  // namespace

extern "C" size_t mars_decode_workspace_bytes(int32_t S, int32_t B, int32_t n_q_heads,
                                              int32_t n_kv_heads, int32_t head_dim,
                                              int32_t page_size, int32_t max_pages) {
  if (!decode_sizes_ok(S, B, n_q_heads, n_kv_heads, head_dim, page_size, max_pages)) return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  return decode_ws_bytes(S, B, n_q_heads, n_kv_heads, head_dim, page_size, max_pages, nullptr,
                         nullptr);
}

extern "C" int mars_attn_block_decode(const void* q, const void* k_new, const void* v_new,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* cache_len,
                                      void* o, int32_t S, int32_t B, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                      int32_t max_pages, int32_t num_pages, int32_t dtype,
                                      float softmax_scale, void* workspace,
                                      size_t workspace_bytes, int32_t* status, void* stream) {
  MARS_REQUIRE(q && k_new && v_new && k_cache && v_cache && block_table && cache_len && o,
               MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_F32 || dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(num_pages >= 1, MARS_ERR_SHAPE);
  MARS_REQUIRE(decode_sizes_ok(S, B, n_q_heads, n_kv_heads, head_dim, page_size, max_pages),
               MARS_ERR_SHAPE);
  MARS_REQUIRE(dtype == MARS_BF16, MARS_ERR_UNSUPPORTED);
  MARS_REQUIRE(head_dim == 64 || head_dim == 128, MARS_ERR_UNSUPPORTED);
  MARS_REQUIRE(mars_aligned16(q) && mars_aligned16(k_new) && mars_aligned16(v_new) &&
                   mars_aligned16(k_cache) && mars_aligned16(v_cache) &&
                   mars_aligned16(block_table) && mars_aligned16(cache_len) &&
                   mars_aligned16(o) && mars_aligned16(workspace),
               MARS_ERR_ALIGN);
  int nsplit = 0, nrows_pad = 0;
  const size_t need = decode_ws_bytes(S, B, n_q_heads, n_kv_heads, head_dim, page_size,
                                      max_pages, &nsplit, &nrows_pad);
  MARS_REQUIRE(workspace && workspace_bytes >= need, MARS_ERR_WORKSPACE);

  DecodeArgs a;
  a.q = (const bf16_t*)q;
  a.k_new = (const bf16_t*)k_new;
  a.v_new = (const bf16_t*)v_new;
  a.k_cache = (const bf16_t*)k_cache;
  a.v_cache = (const bf16_t*)v_cache;
  a.block_table = block_table;
  a.cache_len = cache_len;
  a.o = (bf16_t*)o;
  const size_t rows = (size_t)S * n_kv_heads * nsplit * nrows_pad;
  const size_t ob_al = (rows * head_dim * sizeof(float) + 255) & ~(size_t)255;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + ob_al);
  a.status = status;
  a.S = S;
  a.B = B;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.group = n_q_heads / n_kv_heads;
  a.page_size = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.nsplit = nsplit;
  a.nrows_pad = nrows_pad;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  a.scale_log2 = scale * kLog2e;

  hipStream_t st = (hipStream_t)stream;
  const int nqt = nrows_pad / 32;
  const int merge_waves = S * n_kv_heads * a.group * B;
  dim3 grid(nsplit, n_kv_heads, S);
  if (head_dim == 128) {
    hipLaunchKernelGGL(decode_split_kernel<128>, grid, dim3(64 * nqt), 0, st, a);
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3((merge_waves + 3) / 4), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<64>, grid, dim3(64 * nqt), 0, st, a);
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3((merge_waves + 3) / 4), dim3(256), 0, st, a);
  }
  return mars_launch_status();
}
