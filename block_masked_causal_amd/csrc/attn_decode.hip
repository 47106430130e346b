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
//     operand of lane (dim, hf) is one 16-byte read of 8 consecutive slots
//     (the probabilities are regrouped between the wave halves to match).
// The cache of one sequence is cut into chunks (split-K). Each workgroup
// handles one (chunk, KV head, sequence); when the packed rows fill fewer than
// 4 query tiles, the spare waves of the workgroup split the chunk's keys (4
// waves per tile with one tile, 2 with two, each streaming 512 keys), and
// combine their (max, sum, O) through LDS in a fixed order. Each wave fetches
// the page ids of its own keys. The workgroup
// writes an unnormalised partial (O, running max, running sum) per chunk; a
// merge kernel combines the chunks, and a sequence that fits in one chunk is
// written out directly.
// Chunk 0 also handles the new rows (causal among themselves); the workgroup
// stages their V rows transposed in LDS. Their number may differ per sequence
// (at most 64): under the batch-synchronous block cache (notes, key design 4)
// a sequence's new rows are its tokens accepted since the last frozen block
// followed by the B masks. Packed rows beyond kMaxQT query tiles go to further
// workgroups of the same (chunk, KV head, sequence), which read the same K/V.
#include "mars_common.hpp"

using namespace mars;

namespace {

constexpr int kMaxQT = 4;    // query tiles of 32 packed rows per workgroup
// Waves that share one query tile and split its chunk's keys: a workgroup has
// at most 4 waves, so 1 tile -> 4 key parts, 2 tiles -> 2, 3 or 4 tiles -> 1.
inline int key_split(int nqt) {
  const int t = nqt < kMaxQT ? nqt : kMaxQT;
  return t == 1 ? 4 : t == 2 ? 2 : 1;
}
constexpr int kMaxRows = 64; // new rows per sequence

struct DecodeArgs {
  const bf16_t* q;
  const bf16_t* k_new;
  const bf16_t* v_new;
  const bf16_t* k_cache;
  const bf16_t* v_cache;
  const int32_t* block_table;
  const int32_t* cache_len;
  const int32_t* n_rows;  // NULL: every sequence has B new rows; else n_rows[s] (<= B)
  bf16_t* o;
  float* part_o;   // [S][Hkv][nsplit][nrows_pad][D]
  float* part_ml;  // [S][Hkv][nsplit][nrows_pad][2]
  int32_t* status;
  int S, B, Hq, Hkv, group, page_size, max_pages, num_pages, nsplit, nrows_pad, chunk;
  int qgroups;  // workgroups (of kMaxQT query tiles) per (chunk, KV head, sequence)
  float scale_log2;
};

// One 32-key step for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// Lane (j, hf) holds the scores of packed query row j against step keys
// 8*(r/4) + 4*hf + r%4; MASKED keeps only the keys whose bit is set in `live`.
// Scores of one 32-key step: lane (j, hf) gets packed query row j against
// step keys 8*(r/4) + 4*hf + r%4.
template <int D>
__device__ __forceinline__ f32x16 dec_scores(const bf16x8 (&ka)[D / 16],
                                             const bf16x8* __restrict__ qlds) {
  f32x16 sc = f32x16{};
#pragma unroll
  for (int c = 0; c < D / 16; ++c) sc = mfma32(ka[c], qlds[64 * c], sc);
  return sc;
}

// Online softmax of one step; MASKED keeps only keys whose bit is set in `live`.
template <int D, bool MASKED>
__device__ __forceinline__ void dec_softmax(f32x16& sc, bf16x8 (&pb)[2], f32x16 (&o)[D / 32],
                                            float& m, float& l, float cs, uint32_t live,
                                            int hf) {
  if (MASKED) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
      sc[r] = (live >> key) & 1u ? sc[r] : -INFINITY;
    }
  }
  float mt = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[r]);
  mt = fmaxf(mt, __shfl_xor(mt, 32)) * cs;
  // deferred rescaling: only when a row maximum grows by more than 2^8
  const bool grow = mt > m + 8.0f;
  if (__ballot(grow)) {
    const float mnew = grow ? mt : m;
    const float alpha = m == mnew ? 1.f : fast_exp2(m - mnew);  // -inf - -inf is NaN
    l *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
    m = mnew;
  }
  const float nm = m == -INFINITY ? 0.f : -m;
  float rsum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float e = fast_exp2(fmaf(sc[r], cs, nm));
    rsum += e;
    pb[r >> 3][r & 7] = (bf16_t)e;
  }
  l += rsum;
  // pb[kc] holds keys 16kc + 4hf + (0..3) and 16kc + 8 + 4hf + (0..3). The two
  // wave halves swap dwords 2-3 (half 0) with dwords 0-1 (half 1), so that half
  // hf holds keys 16kc + 8hf + (0..7) in order: the V^T operand of those keys
  // is then one 16-byte read of consecutive slots.
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const u32x4 w = __builtin_bit_cast(u32x4, pb[kc]);
    const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    const u32x4 x = {a[0], b[0], a[1], b[1]};
    pb[kc] = __builtin_bit_cast(bf16x8, x);
  }
}

template <int D>
__device__ __forceinline__ void dec_pv(const bf16x8 (&va)[D / 32][2], const bf16x8 (&pb)[2],
                                       f32x16 (&o)[D / 32]) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] = mfma32(va[i][kc], pb[kc], o[i]);
}

// One complete step (used for the B new rows).
template <int D, bool MASKED>
__device__ __forceinline__ void dec_step(const bf16x8 (&ka)[D / 16], const bf16x8 (&va)[D / 32][2],
                                         const bf16x8* __restrict__ qlds, f32x16 (&o)[D / 32],
                                         float& m, float& l, float cs, uint32_t live, int hf) {
  f32x16 sc = dec_scores<D>(ka, qlds);
  bf16x8 pb[2];
  dec_softmax<D, MASKED>(sc, pb, o, m, l, cs, live, hf);
  dec_pv<D>(va, pb, o);
}

// Keeps the first n (0..8) bf16 values of an 8-key V group, zeroes the rest
// (word masks: element 2w + 1 is the high half of word w).
__device__ __forceinline__ bf16x8 keep_first(bf16x8 v, int n) {
  u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] &= n >= 2 * k + 2 ? 0xFFFFFFFFu : n == 2 * k + 1 ? 0x0000FFFFu : 0u;
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ int rows_of(const DecodeArgs& p, int s) {
  return p.n_rows ? min(max(p.n_rows[s], 0), p.B) : p.B;
}

// Keys of the cache one wave streams: 512 when several waves share a query
// tile (2048-key chunks with four, 1024 with two, so fewer chunk partials are
// written and merged), else 256. A chunk is keys_per_wave x KS keys. A wave's
// keys span at most 32 pages, one page id per lane.
__host__ __device__ constexpr int keys_per_wave(int KS) { return KS == 1 ? 256 : 512; }
// V rows of the new keys (at most kMaxRows) staged transposed in LDS:
// [head_dim][kNewStride] bf16; a row of 144 bytes keeps 16-byte reads aligned.
constexpr int kNewStride = 72;

// Bytes of dynamic LDS of one split workgroup: per wave its query tile (D x 64
// bytes), and the staged V^T of the new rows; the combine of the KS waves of a
// tile reuses that space once the waves are done with it.
__host__ __device__ constexpr size_t split_lds_bytes(int D, int tiles, int KS) {
  const size_t qv = (size_t)tiles * KS * D * 64 + (size_t)D * kNewStride * 2;
  const size_t comb = (size_t)(KS == 4 ? 2 : KS == 2 ? 1 : 0) * tiles * (D / 32 * 16 + 2) * 64 * 4;
  return qv > comb ? qv : comb;
}

// Split-K chunk (cache keys per workgroup): each of the key_split(nqt) waves
// of a query tile streams keys_per_wave of it.
inline int decode_chunk(int nqt) { return keys_per_wave(key_split(nqt)) * key_split(nqt); }

// PS = the page size when it is a compile-time constant (16 or 32, the block
// granularities the method uses), or 0 for any other multiple of 16.
// KS = waves that share one query tile and split its chunk's keys between
// them (1, 2 or 4); a workgroup holds `tiles` query tiles x KS waves.
template <int D, int PS, int KS>
__global__ __launch_bounds__(64 * kMaxQT, 2) void decode_split_kernel(DecodeArgs p) {
  const int split = blockIdx.x, s = blockIdx.z;
  const int kvh = blockIdx.y / p.qgroups, qg = blockIdx.y % p.qgroups;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tiles = (int)blockDim.x / (64 * KS);
  const int wq = w % tiles, kp = w / tiles;  // query tile, key part
  const int j = lane & 31, hf = lane >> 5;
  const int rs = rows_of(p, s);  // new rows of this sequence
  const int nrows = p.group * rs;
  const int tq = qg * kMaxQT + wq;  // this wave's query tile
  // a tile without rows (a sequence with fewer new rows) skips the work but
  // still takes part in the workgroup's barriers
  const bool tile_live = tq * 32 < nrows;

  int len = p.cache_len[s];
  const int cap = p.max_pages * p.page_size;
  if (len > cap) {
    if (split == 0 && kvh == 0 && threadIdx.x == 0) status_or(p.status, MARS_STATUS_CACHE_OVERFLOW);
    len = cap;
  }
  if (len < 0) len = 0;
  const int k_lo = split * p.chunk;
  if (split > 0 && k_lo >= len) return;  // workgroup-uniform
  const int k_hi = min(len, k_lo + p.chunk);
  const bool single = len <= p.chunk;  // the only chunk: write the final output
  // this wave's share of the chunk
  const int w_lo = min(k_lo + kp * keys_per_wave(KS), k_hi);
  const int w_hi = min(w_lo + keys_per_wave(KS), k_hi);

  // Packed query row of this lane: j' = r * g + head_in_group.
  const int qi = tq * 32 + j;
  const bool qvalid = qi < nrows;
  const int qr = qvalid ? qi / p.group : 0;
  const int qh = kvh * p.group + (qvalid ? qi % p.group : 0);
  extern __shared__ bf16x8 qsh[];  // [waves][D / 16][64], then V^T of the new rows
  bf16x8* qlds = qsh + (size_t)w * (D / 16) * 64 + lane;
  bf16_t* vnew = (bf16_t*)(qsh + (size_t)tiles * KS * (D / 16) * 64);
  if (split == 0) {
    // Chunk 0 also attends to the new rows: the workgroup stages their V rows
    // transposed ([d][key], keys rounded up to a multiple of 32, zero past
    // rs), so that the V^T operand of 8 consecutive keys is one 16-byte read.
    const int keys = (rs + 31) & ~31;
    for (int idx = threadIdx.x; idx < keys * (D / 8); idx += blockDim.x) {
      const int t = idx / (D / 8), c = idx % (D / 8);
      u32x4 x = u32x4{0, 0, 0, 0};
      if (t < rs)
        x = *(const u32x4*)(p.v_new + (((size_t)s * p.B + t) * p.Hkv + kvh) * D + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *(uint16_t*)(vnew + (size_t)(8 * c + e) * kNewStride + t) =
            (uint16_t)(x[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();  // workgroup-uniform (split == 0)
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  if (tile_live) {
    {
      const bf16_t* qrow = p.q + (((size_t)s * p.B + qr) * p.Hq + qh) * D + 8 * hf;
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        qlds[64 * c] = qvalid ? *(const bf16x8*)(qrow + 16 * c) : bf16x8{};
    }

    // Page ids of this wave's keys, one per lane (lane t: page w_lo / ps + t;
    // at most 32 pages of >= 16 keys); -1 = bad.
    const int ps = PS > 0 ? PS : p.page_size;
    const int pg0 = w_lo / ps;
    const int npg = w_hi > w_lo ? (w_hi - 1) / ps - pg0 + 1 : 0;
    int mypage = 0;
    if (lane < npg) {
      const int raw = p.block_table[(size_t)s * p.max_pages + pg0 + lane];
      mypage = (raw >= 0 && raw < p.num_pages) ? raw : -1;
    }
    // a wave whose keys touch a bad page masks every step (the page's keys drop out)
    const bool chunk_bad = __ballot(mypage < 0) != 0;
    if (chunk_bad && lane == 0) status_or(p.status, MARS_STATUS_BAD_PAGE);

    const size_t kpage = (size_t)p.Hkv * ps * D;  // elements per page (all heads)
    const bf16_t* kbase = p.k_cache + (size_t)kvh * ps * D;
    const bf16_t* vbase = p.v_cache + (size_t)kvh * D * ps;

    // The step loop is rotated so that a wave always has loads in flight: the K
    // rows of step s+1 are requested as soon as the score MFMAs of step s have
    // consumed the K registers, and the V rows of step s+1 as soon as the PV
    // MFMAs of step s have consumed the V registers.
    bf16x8 ka[D / 16];
    bf16x8 va[D / 32][2];
    auto load_k = [&](int c0) {
      const int pos = c0 + j;
      const int pk = __shfl(mypage, pos / ps - pg0);
      const bf16_t* kr = kbase + (size_t)max(pk, 0) * kpage + (size_t)(pos % ps) * D + 8 * hf;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) ka[c] = *(const bf16x8*)(kr + 16 * c);
    };
    // V group of 8 keys starting at step offset 16kc + 8hf (one page: pages
    // hold a multiple of 16 slots)
    auto v_page = [&](int c0, int kc) {
      return __shfl(mypage, (c0 + 16 * kc + 8 * hf) / ps - pg0);
    };
    auto load_v = [&](int c0) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int k0 = c0 + 16 * kc + 8 * hf;
        const bf16_t* v0 = vbase + (size_t)max(v_page(c0, kc), 0) * kpage + (k0 % ps);
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
          va[i][kc] = *(const bf16x8*)(v0 + (size_t)(32 * i + j) * ps);
      }
    };
    // A step that masks keys past the wave's end or on a bad page (their V
    // slots are zeroed too: stale slots may hold anything); K and V loaded.
    auto masked_step = [&](int c0) {
      f32x16 sc = dec_scores<D>(ka, qlds);
      const int pos = c0 + j;
      const uint32_t live =
          (uint32_t)__ballot(pos < w_hi && __shfl(mypage, pos / ps - pg0) >= 0);
      bf16x8 pb[2];
      dec_softmax<D, true>(sc, pb, o, m, l, p.scale_log2, live, hf);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int k0 = c0 + 16 * kc + 8 * hf;
        const int n0 = v_page(c0, kc) < 0 ? 0 : w_hi - k0;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) va[i][kc] = keep_first(va[i][kc], n0);
      }
      dec_pv<D>(va, pb, o);
    };
    if (!chunk_bad) {
      // whole 32-key steps, then at most one partial step: keeping the masked
      // code out of the loop keeps its registers out of the loop's live set
      const int w_full = w_lo + ((w_hi - w_lo) & ~31);
      if (w_lo < w_hi) {
        load_k(w_lo);
        load_v(w_lo);
      }
      for (int c0 = w_lo; c0 < w_full; c0 += 32) {
        const bool more = c0 + 32 < w_hi;
        f32x16 sc = dec_scores<D>(ka, qlds);
        __builtin_amdgcn_sched_barrier(0);
        if (more) load_k(c0 + 32);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 pb[2];
        dec_softmax<D, false>(sc, pb, o, m, l, p.scale_log2, 0u, hf);
        dec_pv<D>(va, pb, o);
        __builtin_amdgcn_sched_barrier(0);
        if (more) load_v(c0 + 32);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (w_full < w_hi) masked_step(w_full);
    } else {
      for (int c0 = w_lo; c0 < w_hi; c0 += 32) {
        load_k(c0);
        load_v(c0);
        masked_step(c0);
      }
    }

    // ---- the new rows, causal among themselves (chunk 0, last key part) ----
    if (split == 0 && kp == KS - 1) {
      for (int n0 = 0; n0 < rs; n0 += 32) {
        {
          const bool kv = n0 + j < rs;
          const bf16_t* kr =
              p.k_new + (((size_t)s * p.B + (kv ? n0 + j : 0)) * p.Hkv + kvh) * D + 8 * hf;
#pragma unroll
          for (int c = 0; c < D / 16; ++c) ka[c] = kv ? *(const bf16x8*)(kr + 16 * c) : bf16x8{};
        }
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int kc = 0; kc < 2; ++kc)
            va[i][kc] = *(const bf16x8*)(vnew + (size_t)(32 * i + j) * kNewStride + n0 +
                                         16 * kc + 8 * hf);
        // new row n0 + t is visible to packed row j' iff n0 + t <= r(j'): a per-lane mask
        const int vis = qr - n0 + 1;  // visible keys of this step
        const uint32_t live = vis <= 0 ? 0u : vis >= 32 ? 0xFFFFFFFFu : ((1u << vis) - 1u);
        dec_step<D, true>(ka, va, qlds, o, m, l, p.scale_log2, live, hf);
      }
    }
  }

  // ---- the KS waves of a tile combine, in a fixed order -------------------
  if constexpr (KS > 1) {
    constexpr int kOF = D / 32 * 16 * 64;  // floats of one wave's O
    float* cbuf = (float*)qsh;             // reuses the query and staging space
    auto slot = [&](int k) { return cbuf + (size_t)(k * tiles + wq) * (kOF + 128); };
    auto put = [&](float* b) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) b[(i * 16 + r) * 64 + lane] = o[i][r];
      b[kOF + lane] = m;
      b[kOF + 64 + lane] = l;
    };
    // (m, l, O) of this wave and of the wave that wrote b, in that order
    auto take = [&](const float* b) {
      const float mb = b[kOF + lane], lb = b[kOF + 64 + lane];
      const float M = fmaxf(m, mb);
      const float sa = m == M ? 1.f : fast_exp2(m - M);
      const float sb = mb == M ? 1.f : fast_exp2(mb - M);
      l = l * sa + lb * sb;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] = o[i][r] * sa + b[(i * 16 + r) * 64 + lane] * sb;
      m = M;
    };
    __syncthreads();  // every wave is done with the query and staging space
    if (KS == 4) {    // ((0 + 1) + (2 + 3))
      if (kp & 1) put(slot(kp >> 1));
      __syncthreads();
      if (!(kp & 1)) take(slot(kp >> 1));
      __syncthreads();
      if (kp == 2) put(slot(0));
      __syncthreads();
      if (kp == 0) take(slot(0));
    } else {  // (0 + 1)
      if (kp == 1) put(slot(0));
      __syncthreads();
      if (kp == 0) take(slot(0));
    }
    if (kp != 0) return;
  }
  if (!tile_live) return;

  // ---- partial result for this chunk ---------------------------------------
  const float lt = l + __shfl_xor(l, 32);
  if (!qvalid) return;
  if (single) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    bf16_t* orow = p.o + (((size_t)s * p.B + qr) * p.Hq + qh) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk = {pack_bf16x2(o[i][4 * g] * inv, o[i][4 * g + 1] * inv),
                    pack_bf16x2(o[i][4 * g + 2] * inv, o[i][4 * g + 3] * inv)};
        *(u32x2*)(orow + 32 * i + 8 * g + 4 * hf) = pk;
      }
    return;
  }
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

// One workgroup per (sequence, KV head): combine the chunks of each packed
// query row. A thread owns 4 consecutive head-dimension elements of a row at a
// time (D / 4 threads per row); a sequence whose cache fits in one chunk was
// written directly by the split kernel and is skipped.
constexpr int kMergeThreads = 512;
template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs p) {
  const int kvh = blockIdx.x % p.Hkv;
  const int s = blockIdx.x / p.Hkv;
  int len = p.cache_len[s];
  len = min(max(len, 0), p.max_pages * p.page_size);
  const int nsp = max(1, (len + p.chunk - 1) / p.chunk);
  if (nsp == 1) return;  // written directly by the split kernel
  const int nrows = p.group * rows_of(p, s);
  constexpr int Q4 = D / 4;  // threads per row
  const size_t stride = p.nrows_pad;
  const size_t base0 = ((size_t)s * p.Hkv + kvh) * p.nsplit * p.nrows_pad;
  // Chunks are taken kMergeBatch at a time with all their loads in flight
  // (one memory round trip per batch, not two per chunk), in chunk order. A
  // later batch that raises the maximum rescales what came before; with at
  // most kMergeBatch chunks the arithmetic is a single fixed-order pass.
  constexpr int kMergeBatch = 8;
  for (int e = threadIdx.x; e < nrows * Q4; e += kMergeThreads) {
    const int qi = e / Q4, d0 = 4 * (e % Q4);
    const size_t base = base0 + qi;
    float M = -INFINITY, lsum = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < nsp; sp0 += kMergeBatch) {
      float mv[kMergeBatch], lv[kMergeBatch];
      f32x4 ov[kMergeBatch];
#pragma unroll
      for (int t = 0; t < kMergeBatch; ++t) {
        const bool in = sp0 + t < nsp;
        const size_t row = base + (size_t)(in ? sp0 + t : sp0) * stride;
        mv[t] = in ? p.part_ml[row * 2] : -INFINITY;
        lv[t] = in ? p.part_ml[row * 2 + 1] : 0.f;
        ov[t] = in ? *(const f32x4*)(p.part_o + row * D + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float mt = M;
#pragma unroll
      for (int t = 0; t < kMergeBatch; ++t) mt = fmaxf(mt, mv[t]);
      const float mb = mt == -INFINITY ? 0.f : mt;
      if (M != -INFINITY && M != mt) {  // a later batch raised the maximum
        const float sc = fast_exp2(M - mb);
        lsum *= sc;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] *= sc;
      }
#pragma unroll
      for (int t = 0; t < kMergeBatch; ++t) {
        const float w = mv[t] == -INFINITY ? 0.f : fast_exp2(mv[t] - mb);
        lsum += w * lv[t];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] += w * ov[t][k];
      }
      M = mt;
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int r = qi / p.group, h = kvh * p.group + qi % p.group;
    bf16_t* orow = p.o + (((size_t)s * p.B + r) * p.Hq + h) * D + d0;
    *(u32x2*)orow = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                          pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  }
}

size_t decode_ws_bytes(int S, int B, int Hq, int Hkv, int D, int page_size, int max_pages,
                       int* nsplit_out, int* nrows_pad_out) {
  const long long cap = (long long)max_pages * page_size;
  const int nrows = (Hq / Hkv) * B;
  const int nrows_pad = ((nrows + 31) / 32) * 32;
  const int chunk = decode_chunk(nrows_pad / 32);
  const int nsplit = (int)std::max<long long>(1, (cap + chunk - 1) / chunk);
  if (nsplit_out) *nsplit_out = nsplit;
  if (nrows_pad_out) *nrows_pad_out = nrows_pad;
  const size_t rows = (size_t)S * Hkv * nsplit * nrows_pad;
  const size_t ob = rows * D * sizeof(float);
  const size_t ob_al = (ob + 255) & ~(size_t)255;
  return ob_al + rows * 2 * sizeof(float);
}

bool decode_sizes_ok(int S, int B, int Hq, int Hkv, int D, int page_size, int max_pages) {
  if (S < 1 || B < 1 || B > kMaxRows || Hq < 1 || Hkv < 1 || Hq % Hkv) return false;
  if (Hq > 4096) return false;
  const int nqt = ((Hq / Hkv) * B + 31) / 32;
  if ((long long)Hkv * ((nqt + kMaxQT - 1) / kMaxQT) > 65535) return false;
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

namespace {
// Common path of both entry points; n_rows NULL means B rows for every sequence.
int run_decode(const void* q, const void* k_new, const void* v_new, const void* k_cache,
               const void* v_cache, const int32_t* block_table, const int32_t* cache_len,
               const int32_t* n_rows, void* o, int32_t S, int32_t B, int32_t n_q_heads,
               int32_t n_kv_heads, int32_t head_dim, int32_t page_size, int32_t max_pages,
               int32_t num_pages, int32_t dtype, float softmax_scale, void* workspace,
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
                   mars_aligned16(o) && mars_aligned16(workspace) && mars_aligned16(n_rows),
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
  a.n_rows = n_rows;
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
  a.chunk = decode_chunk(nrows_pad / 32);
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  a.scale_log2 = scale * kLog2e;

  hipStream_t st = (hipStream_t)stream;
  const int nqt = nrows_pad / 32;
  const int wg_tiles = nqt < kMaxQT ? nqt : kMaxQT;
  a.qgroups = (nqt + kMaxQT - 1) / kMaxQT;
  const long long merge_blocks = (long long)S * n_kv_heads;
  MARS_REQUIRE(merge_blocks < (1LL << 31), MARS_ERR_SHAPE);
  dim3 grid(nsplit, n_kv_heads * a.qgroups, S);
  const int ks = key_split(nqt);
  const size_t lds = split_lds_bytes(head_dim, wg_tiles, ks);
  const dim3 blk(64 * wg_tiles * ks);
#define MARS_DECODE_LAUNCH(D_, PS_)                                                           \
  do {                                                                                        \
    if (ks == 4)                                                                              \
      hipLaunchKernelGGL((decode_split_kernel<D_, PS_, 4>), grid, blk, lds, st, a);           \
    else if (ks == 2)                                                                         \
      hipLaunchKernelGGL((decode_split_kernel<D_, PS_, 2>), grid, blk, lds, st, a);           \
    else                                                                                      \
      hipLaunchKernelGGL((decode_split_kernel<D_, PS_, 1>), grid, blk, lds, st, a);           \
  } while (0)
  if (head_dim == 128) {
    if (page_size == 16) MARS_DECODE_LAUNCH(128, 16);
    else if (page_size == 32) MARS_DECODE_LAUNCH(128, 32);
    else MARS_DECODE_LAUNCH(128, 0);
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3((unsigned)merge_blocks), dim3(kMergeThreads), 0, st, a);
  } else {
    if (page_size == 16) MARS_DECODE_LAUNCH(64, 16);
    else if (page_size == 32) MARS_DECODE_LAUNCH(64, 32);
    else MARS_DECODE_LAUNCH(64, 0);
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3((unsigned)merge_blocks), dim3(kMergeThreads), 0, st, a);
  }
#undef MARS_DECODE_LAUNCH
  return mars_launch_status();
}
}  // namespace

extern "C" int mars_attn_block_decode(const void* q, const void* k_new, const void* v_new,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* cache_len,
                                      void* o, int32_t S, int32_t B, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                      int32_t max_pages, int32_t num_pages, int32_t dtype,
                                      float softmax_scale, void* workspace,
                                      size_t workspace_bytes, int32_t* status, void* stream) {
  return run_decode(q, k_new, v_new, k_cache, v_cache, block_table, cache_len, nullptr, o, S,
                    B, n_q_heads, n_kv_heads, head_dim, page_size, max_pages, num_pages, dtype,
                    softmax_scale, workspace, workspace_bytes, status, stream);
}

extern "C" int mars_attn_block_decode_rows(const void* q, const void* k_new, const void* v_new,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* block_table,
                                           const int32_t* cache_len, const int32_t* n_rows,
                                           void* o, int32_t S, int32_t R, int32_t n_q_heads,
                                           int32_t n_kv_heads, int32_t head_dim,
                                           int32_t page_size, int32_t max_pages,
                                           int32_t num_pages, int32_t dtype,
                                           float softmax_scale, void* workspace,
                                           size_t workspace_bytes, int32_t* status,
                                           void* stream) {
  MARS_REQUIRE(n_rows, MARS_ERR_NULL);
  return run_decode(q, k_new, v_new, k_cache, v_cache, block_table, cache_len, n_rows, o, S, R,
                    n_q_heads, n_kv_heads, head_dim, page_size, max_pages, num_pages, dtype,
                    softmax_scale, workspace, workspace_bytes, status, stream);
}
