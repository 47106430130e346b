// Left-to-right acceptance + KV commit for gfx950.
//
// Acceptance follows the papernotes.org notes on "MARS: Enabling Autoregressive
// Models Multi-Token Generation", key design 3 (关键设计 3), and the
// gist.science explainer, section 2C: scan the B positions left to right,
// accept while the max-probability is at least tau, stop at the first position
// below tau, and always accept the first. The accepted tokens then join the
// persistent prefix KV cache (notes, key design 4 / 关键设计 4).
//
// One workgroup per sequence. Wave 0 takes the decision with one lane per
// position (a ballot of p >= tau; the accepted count is the run of passing
// positions from the first) and resolves the destination page of each
// committed row in parallel; then the whole workgroup copies the accepted
// rows: K rows as 16-byte vectors into the [page][head][slot][d] pages, V rows
// element-wise into the transposed [page][head][d][slot] pages, with
// consecutive threads on consecutive slots.
#include "mars_common.hpp"

using namespace mars;

namespace {

constexpr int kMaxB = 64;

struct CommitArgs {
  const float* p_max;
  const int32_t* top_id;
  const float* tau;
  const char* k_new;
  const char* v_new;
  char* k_cache;
  char* v_cache;
  const int32_t* block_table;
  int32_t* cache_len;
  int32_t* n_accepted;
  int32_t* accepted_ids;
  int32_t* commit_pos;
  int32_t* status;
  int S, B, Hkv, D, page_size, max_pages, num_pages;
  int layers;  // caches and new rows hold this many layers, back to back
};

// Accepted count of one row of B max-probabilities: the leading run of
// p >= tau (a NaN compares false and stops the run), at least 1.
__device__ __forceinline__ int accepted_count(const float* pr, int B, float tau) {
  int n = 0;
  while (n < B && pr[n] >= tau) ++n;
  return n < 1 ? 1 : n;
}

// The decision of sequence s, taken by one whole wave with lane r = position
// r: the accepted count is the run of set bits at the bottom of the ballot of
// p >= tau (a NaN compares false), at least 1; each accepted row resolves its
// page in parallel and the commit keeps the rows before the first one that
// cannot be placed. Writes n_accepted, accepted_ids, commit_pos and the first
// failure's status flag; returns the rows placed (nc) and the old length, and
// the page of row r in *pg (rows r < nc).
__device__ __forceinline__ int decide(const CommitArgs& p, int s, int r, int* len_out, int* pg_out) {
  const bool pass = r < p.B && p.p_max[(size_t)s * p.B + r] >= p.tau[s];
  const uint64_t pm = __ballot(pass);
  const int n = max(pm == ~0ull ? 64 : __builtin_ctzll(~pm), 1);
  const int len = p.cache_len[s];
  const long long cap = (long long)p.max_pages * p.page_size;
  int pg = -1;
  int32_t flag = 0;
  if (r < n) {
    const long long pos = (long long)len + r;
    if (len < 0 || pos >= cap) {
      flag = MARS_STATUS_CACHE_OVERFLOW;
    } else {
      pg = p.block_table[(size_t)s * p.max_pages + (int)(pos / p.page_size)];
      if (pg < 0 || pg >= p.num_pages) flag = MARS_STATUS_BAD_PAGE;
    }
  }
  const uint64_t gm = __ballot(r < n && flag == 0);
  const int nc = gm == ~0ull ? 64 : __builtin_ctzll(~gm);  // rows placed
  if (r == nc && r < n) status_or(p.status, flag);          // the first failure
  if (r < p.B) {
    p.accepted_ids[(size_t)s * p.B + r] = r < n ? p.top_id[(size_t)s * p.B + r] : -1;
    p.commit_pos[(size_t)s * p.B + r] = r < nc ? len + r : -1;
  }
  if (r == 0) p.n_accepted[s] = n;
  *len_out = len;
  *pg_out = pg;
  return nc;
}

constexpr int kCommitStageBytes = 16384;  // LDS staging of V rows in the commit

// Copies rows 0 .. nc-1 of sequence s of one layer (the rows' pages in
// page[r], positions len + r) into that layer's caches; every thread of the
// 256-thread workgroup takes part. K rows go as 16-byte vectors into the
// [page][head][slot][d] pages, head-major so that the rows of one head land
// on consecutive slots. V rows: the (head, row) pairs are staged in LDS
// (head-major, with 16-byte loads: a row is contiguous in v_new), then
// written to the transposed [page][head][d][slot] pages one element per
// thread, row fastest, so that neighbouring lanes store neighbouring slots.
// Rows too long for the staging buffer take the element path directly.
template <int ES>  // element size in bytes (2 = bf16, 4 = fp32)
__device__ __forceinline__ void copy_rows(const CommitArgs& p, int layer, int s, int len, int nc,
                                          const int* page, char* vst) {
  const int tid = threadIdx.x;
  const int rowbytes = p.D * ES;  // one head's row
  const int chunks = rowbytes / 16;
  const size_t new_off = (size_t)layer * p.S * p.B * p.Hkv * rowbytes;
  const size_t cache_off = (size_t)layer * p.num_pages * p.Hkv * p.page_size * rowbytes;
  const char* k_new = p.k_new + new_off;
  const char* v_new = p.v_new + new_off;
  char* k_cache = p.k_cache + cache_off;
  char* v_cache = p.v_cache + cache_off;

  for (int idx = tid; idx < nc * p.Hkv * chunks; idx += 256) {
    const int ch = idx % chunks;
    const int r = (idx / chunks) % nc;
    const int kvh = idx / (chunks * nc);
    const int pos = len + r;
    const size_t src = (((size_t)s * p.B + r) * p.Hkv + kvh) * rowbytes + ch * 16;
    const size_t dst =
        (((size_t)page[r] * p.Hkv + kvh) * p.page_size + pos % p.page_size) * rowbytes + ch * 16;
    *(u32x4*)(k_cache + dst) = *(const u32x4*)(k_new + src);
  }
  const int vrs = rowbytes + 4;  // padded LDS row stride
  const int rows = nc * p.Hkv;   // staged (head, row) pairs, j = head * nc + row
  if (nc > 1 && vrs <= kCommitStageBytes) {
    const int G = kCommitStageBytes / vrs;  // pairs per pass
    for (int j0 = 0; j0 < rows; j0 += G) {
      const int g = min(G, rows - j0);
      for (int idx = tid; idx < g * chunks; idx += 256) {
        const int ch = idx % chunks;
        const int j = j0 + idx / chunks;
        const int r = j % nc, kvh = j / nc;
        const u32x4 x =
            *(const u32x4*)(v_new + (((size_t)s * p.B + r) * p.Hkv + kvh) * rowbytes + ch * 16);
        uint32_t* d4 = (uint32_t*)(vst + (j - j0) * vrs + ch * 16);
        d4[0] = x[0];
        d4[1] = x[1];
        d4[2] = x[2];
        d4[3] = x[3];
      }
      __syncthreads();
      for (int idx = tid; idx < g * p.D; idx += 256) {
        const int jj = idx % g;
        const int d = idx / g;
        const int j = j0 + jj;
        const int r = j % nc, kvh = j / nc;
        const int pos = len + r;
        const size_t dst =
            ((((size_t)page[r] * p.Hkv + kvh) * p.D + d) * p.page_size + pos % p.page_size) * ES;
        if (ES == 2)
          *(uint16_t*)(v_cache + dst) = *(const uint16_t*)(vst + jj * vrs + d * 2);
        else
          *(uint32_t*)(v_cache + dst) = *(const uint32_t*)(vst + jj * vrs + d * 4);
      }
      __syncthreads();
    }
  } else {
    for (int idx = tid; idx < nc * p.Hkv * p.D; idx += 256) {
      const int r = idx % nc;
      const int d = (idx / nc) % p.D;
      const int kvh = idx / (nc * p.D);
      const int pos = len + r;
      const size_t src = ((((size_t)s * p.B + r) * p.Hkv + kvh) * p.D + d) * ES;
      const size_t dst =
          ((((size_t)page[r] * p.Hkv + kvh) * p.D + d) * p.page_size + pos % p.page_size) * ES;
      if (ES == 2)
        *(uint16_t*)(v_cache + dst) = *(const uint16_t*)(v_new + src);
      else
        *(uint32_t*)(v_cache + dst) = *(const uint32_t*)(v_new + src);
    }
    __syncthreads();
  }
}

// One layer: one workgroup per sequence. Wave 0 decides (see decide), then
// the whole workgroup copies the accepted rows and thread 0 advances
// cache_len.
template <int ES>
__global__ __launch_bounds__(256) void accept_commit_kernel(CommitArgs p) {
  __shared__ int sh_page[kMaxB];
  __shared__ int sh_len, sh_nc;
  __shared__ __attribute__((aligned(16))) char vst[kCommitStageBytes];
  const int s = blockIdx.x, tid = threadIdx.x;
  if (tid < 64) {
    int len, pg;
    const int nc = decide(p, s, tid, &len, &pg);
    if (tid < nc) sh_page[tid] = pg;
    if (tid == 0) {
      sh_len = len;
      sh_nc = nc;
    }
  }
  __syncthreads();
  const int len = sh_len, nc = sh_nc;
  copy_rows<ES>(p, 0, s, len, nc, sh_page, vst);
  if (tid == 0) p.cache_len[s] = len + nc;
}

// Several layers, first launch: the decision of 4 sequences per workgroup,
// one wave each; each wave also advances its sequence's cache_len (the copy
// that follows reads the positions from commit_pos, not from cache_len).
__global__ __launch_bounds__(256) void accept_decide_kernel(CommitArgs p) {
  const int s = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int r = threadIdx.x & 63;
  if (s >= p.S) return;  // wave-uniform
  int len, pg;
  const int nc = decide(p, s, r, &len, &pg);
  if (r == 0) p.cache_len[s] = len + nc;
}

// Several layers, second launch: workgroup (s, layer) copies the committed
// rows of sequence s of that layer. The rows are the leading run of
// commit_pos[s, r] == commit_pos[s, 0] + r; each row's page is looked up
// again (and a row whose page is out of range ends the run, which the
// decision already excluded).
template <int ES>
__global__ __launch_bounds__(256) void commit_layers_kernel(CommitArgs p) {
  __shared__ int sh_page[kMaxB];
  __shared__ int sh_len, sh_nc;
  __shared__ __attribute__((aligned(16))) char vst[kCommitStageBytes];
  const int s = blockIdx.x, layer = blockIdx.y, tid = threadIdx.x;
  if (tid < 64) {
    const int r = tid;
    const int len = p.commit_pos[(size_t)s * p.B];
    const long long cap = (long long)p.max_pages * p.page_size;
    bool ok = false;
    int pg = -1;
    if (r < p.B && len >= 0) {
      const int pos = p.commit_pos[(size_t)s * p.B + r];
      if (pos == len + r && (long long)pos < cap) {
        pg = p.block_table[(size_t)s * p.max_pages + pos / p.page_size];
        ok = pg >= 0 && pg < p.num_pages;
      }
    }
    const uint64_t m = __ballot(ok);
    const int nc = m == ~0ull ? 64 : __builtin_ctzll(~m);
    if (r < nc) sh_page[r] = pg;
    if (r == 0) {
      sh_len = len;
      sh_nc = nc;
    }
  }
  __syncthreads();
  copy_rows<ES>(p, layer, s, sh_len, sh_nc, sh_page, vst);
}

// ---------------------------------------------------------------- append ----
// Append T rows per sequence to the paged cache (the prefill's K/V): row r of
// sequence s goes to position cache_len[s] + r. Grid (ceil((T + 7) / 64), S,
// KV heads): workgroup (x, s, h) owns head h of the 64 cache positions
// starting at (cache_len[s] rounded down to a multiple of 8) + 64 x, so that
// every group of 8 positions it writes is 8-aligned. It resolves the page of
// each position in parallel, copies the K rows straight through
// ([page][head][slot][d] keeps a row contiguous), and stages the V rows in LDS
// so that it can write the transposed V layout ([page][head][d][slot]) as runs
// of 8 slots, one 16-byte store per run of 8 bf16 values, where the page size
// is a multiple of 8; other page sizes take element stores.
struct AppendArgs {
  const char* k_rows;
  const char* v_rows;
  char* k_cache;
  char* v_cache;
  const int32_t* block_table;
  int32_t* cache_len;
  int32_t* status;
  const int32_t* gate;  // NULL, or: append only if gate[s] == gate_full for every s
  int gate_full;
  int src_rows;         // rows per sequence in k_rows / v_rows (>= T)
  int S, T, Hkv, D, page_size, max_pages, num_pages;
};

// Whether the gate holds for the whole batch (every thread of the block takes
// part; the result is block-uniform).
__device__ __forceinline__ bool gate_open(const AppendArgs& p) {
  if (!p.gate) return true;
  int ok = 1;
  for (int i = threadIdx.x; i < p.S; i += blockDim.x) ok &= p.gate[i] == p.gate_full;
  return __syncthreads_and(ok) != 0;
}

constexpr int kAppendMaxRowBytes = 512;  // head_dim * element size staged per V row

template <int ES>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs p) {
  // V rows of one head, row stride rowbytes + 4 so that column reads of rows
  // 8 apart fall in different banks
  // (dynamic LDS of 64 * (head_dim * ES + 4) bytes)
  extern __shared__ __attribute__((aligned(16))) char sv[];
  __shared__ int sh_page[64];  // page of each window position; -1 skip (flagged), -2 not ours
  // heads fastest: the workgroups of one window read neighbouring slices of
  // the same source rows
  const int s = blockIdx.y, kvh = blockIdx.x % p.Hkv, win = blockIdx.x / p.Hkv;
  const int tid = threadIdx.x;
  if (!gate_open(p)) return;
  const int len = p.cache_len[s];
  if (len < 0) {
    if (blockIdx.x == 0 && tid == 0) status_or(p.status, MARS_STATUS_CACHE_OVERFLOW);
    return;
  }
  const long long wbase = (long long)(len & ~7) + 64LL * win;
  const long long cap = (long long)p.max_pages * p.page_size;
  if (tid < 64) {
    const long long pos = wbase + tid;
    int pg = -2;
    if (pos >= len && pos < (long long)len + p.T) {
      if (pos >= cap) {
        if (kvh == 0) status_or(p.status, MARS_STATUS_CACHE_OVERFLOW);
        pg = -1;
      } else {
        pg = p.block_table[(size_t)s * p.max_pages + (int)(pos / p.page_size)];
        if (pg < 0 || pg >= p.num_pages) {
          if (kvh == 0) status_or(p.status, MARS_STATUS_BAD_PAGE);
          pg = -1;
        }
      }
    }
    sh_page[tid] = pg;
  }
  __syncthreads();
  const int rowbytes = p.D * ES;
  const int chunks = rowbytes / 16;
  // a position with a page (pg >= 0) lies in [len, min(len + T, cap)): its row
  // index and slot fit in int
  const size_t row0 = (size_t)s * p.src_rows;  // first row of this sequence
  for (int idx = tid; idx < 64 * chunks; idx += 256) {
    const int ch = idx % chunks;
    const int t = idx / chunks;
    const int pg = sh_page[t];
    if (pg < 0) continue;
    const int pos = (int)(wbase + t);
    const size_t src = ((row0 + (pos - len)) * p.Hkv + kvh) * rowbytes + ch * 16;
    const size_t dst =
        (((size_t)pg * p.Hkv + kvh) * p.page_size + pos % p.page_size) * rowbytes + ch * 16;
    *(u32x4*)(p.k_cache + dst) = *(const u32x4*)(p.k_rows + src);
  }
  const int rs = rowbytes + 4;
  const bool runs = (p.page_size % 8) == 0;
  {
    for (int idx = tid; idx < 64 * chunks; idx += 256) {
      const int ch = idx % chunks;
      const int t = idx / chunks;
      if (sh_page[t] < 0) continue;
      const int pos = (int)(wbase + t);
      const u32x4 x = *(const u32x4*)(p.v_rows + ((row0 + (pos - len)) * p.Hkv + kvh) *
                                                     rowbytes + ch * 16);
      uint32_t* d4 = (uint32_t*)(sv + t * rs + ch * 16);
      d4[0] = x[0];
      d4[1] = x[1];
      d4[2] = x[2];
      d4[3] = x[3];
    }
    __syncthreads();
    // (d, group of 8 positions), groups fastest: lanes next to each other
    // write neighbouring slot runs of the same V column
    for (int idx = tid; idx < 8 * p.D; idx += 256) {
      const int g = idx & 7;
      const int d = idx >> 3;
      const int t0 = 8 * g;
      const int pg0 = sh_page[t0];
      bool whole = runs && pg0 >= 0;
#pragma unroll
      for (int i = 1; i < 8; ++i) whole = whole && sh_page[t0 + i] >= 0;
      if (whole) {  // 8 aligned positions of one page: one contiguous run
        const int pos0 = (int)(wbase + t0);
        char* dst = p.v_cache + ((((size_t)pg0 * p.Hkv + kvh) * p.D + d) * p.page_size +
                                 pos0 % p.page_size) * ES;
        if (ES == 2) {
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)*(const uint16_t*)(sv + (t0 + 2 * i) * rs + d * 2) |
                   ((uint32_t)*(const uint16_t*)(sv + (t0 + 2 * i + 1) * rs + d * 2) << 16);
          *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
        } else {
          uint32_t w[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = *(const uint32_t*)(sv + (t0 + i) * rs + d * 4);
          *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
          *(u32x4*)(dst + 16) = u32x4{w[4], w[5], w[6], w[7]};
        }
      } else {
        for (int i = 0; i < 8; ++i) {
          const int pg = sh_page[t0 + i];
          if (pg < 0) continue;
          const int pos = (int)(wbase + t0 + i);
          char* dst = p.v_cache + ((((size_t)pg * p.Hkv + kvh) * p.D + d) * p.page_size +
                                   pos % p.page_size) * ES;
          if (ES == 2)
            *(uint16_t*)dst = *(const uint16_t*)(sv + (t0 + i) * rs + d * 2);
          else
            *(uint32_t*)dst = *(const uint32_t*)(sv + (t0 + i) * rs + d * 4);
        }
      }
    }
  }
}

// After the copy (same stream): cache_len[s] advances by the rows that fit.
__global__ __launch_bounds__(256) void kv_append_len_kernel(AppendArgs p) {
  if (!gate_open(p)) return;
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= p.S) return;
  const int len = p.cache_len[s];
  if (len < 0) return;
  const long long cap = (long long)p.max_pages * p.page_size;
  p.cache_len[s] = (int)min((long long)len + p.T, max((long long)len, cap));
}

}  // namespace

namespace {
// Checks shared by the one-layer and the layered commit, then the kernel
// arguments.
int commit_args(const float* p_max, const int32_t* top_id, const float* tau, const void* k_new,
                const void* v_new, void* k_cache, void* v_cache, const int32_t* block_table,
                int32_t* cache_len, int32_t* n_accepted, int32_t* accepted_ids,
                int32_t* commit_pos, int32_t layers, int32_t S, int32_t B, int32_t n_kv_heads,
                int32_t head_dim, int32_t page_size, int32_t max_pages, int32_t num_pages,
                int32_t dtype, int32_t* status, CommitArgs* a) {
  MARS_REQUIRE(p_max && top_id && tau && k_new && v_new && k_cache && v_cache && block_table &&
                   cache_len && n_accepted && accepted_ids && commit_pos,
               MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_F32 || dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(S >= 1 && S <= (1 << 30) && B >= 1 && B <= kMaxB, MARS_ERR_SHAPE);
  MARS_REQUIRE(layers >= 1 && layers <= 65535, MARS_ERR_SHAPE);
  MARS_REQUIRE(n_kv_heads >= 1 && head_dim >= 8 && head_dim % 8 == 0, MARS_ERR_SHAPE);
  MARS_REQUIRE(page_size >= 1 && max_pages >= 1 && num_pages >= 1, MARS_ERR_SHAPE);
  MARS_REQUIRE((long long)max_pages * page_size <= (1LL << 30), MARS_ERR_SHAPE);
  MARS_REQUIRE(mars_aligned16(p_max) && mars_aligned16(top_id) && mars_aligned16(tau) &&
                   mars_aligned16(k_new) && mars_aligned16(v_new) && mars_aligned16(k_cache) &&
                   mars_aligned16(v_cache) && mars_aligned16(block_table) &&
                   mars_aligned16(cache_len) && mars_aligned16(n_accepted) &&
                   mars_aligned16(accepted_ids) && mars_aligned16(commit_pos),
               MARS_ERR_ALIGN);
  a->p_max = p_max;
  a->top_id = top_id;
  a->tau = tau;
  a->k_new = (const char*)k_new;
  a->v_new = (const char*)v_new;
  a->k_cache = (char*)k_cache;
  a->v_cache = (char*)v_cache;
  a->block_table = block_table;
  a->cache_len = cache_len;
  a->n_accepted = n_accepted;
  a->accepted_ids = accepted_ids;
  a->commit_pos = commit_pos;
  a->status = status;
  a->S = S;
  a->B = B;
  a->Hkv = n_kv_heads;
  a->D = head_dim;
  a->page_size = page_size;
  a->max_pages = max_pages;
  a->num_pages = num_pages;
  a->layers = layers;
  return MARS_OK;
}
}  // namespace

extern "C" int mars_accept_commit(const float* p_max, const int32_t* top_id, const float* tau,
                                  const void* k_new, const void* v_new, void* k_cache,
                                  void* v_cache, const int32_t* block_table, int32_t* cache_len,
                                  int32_t* n_accepted, int32_t* accepted_ids,
                                  int32_t* commit_pos, int32_t S, int32_t B, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t page_size, int32_t max_pages,
                                  int32_t num_pages, int32_t dtype, int32_t* status,
                                  void* stream) {
  CommitArgs a;
  const int rc = commit_args(p_max, top_id, tau, k_new, v_new, k_cache, v_cache, block_table,
                             cache_len, n_accepted, accepted_ids, commit_pos, 1, S, B,
                             n_kv_heads, head_dim, page_size, max_pages, num_pages, dtype, status,
                             &a);
  if (rc != MARS_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == MARS_BF16)
    hipLaunchKernelGGL(accept_commit_kernel<2>, dim3(S), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(accept_commit_kernel<4>, dim3(S), dim3(256), 0, st, a);
  return mars_launch_status();
}

extern "C" int mars_accept_commit_layers(const float* p_max, const int32_t* top_id,
                                         const float* tau, const void* k_new, const void* v_new,
                                         void* k_cache, void* v_cache,
                                         const int32_t* block_table, int32_t* cache_len,
                                         int32_t* n_accepted, int32_t* accepted_ids,
                                         int32_t* commit_pos, int32_t n_layers, int32_t S,
                                         int32_t B, int32_t n_kv_heads, int32_t head_dim,
                                         int32_t page_size, int32_t max_pages,
                                         int32_t num_pages, int32_t dtype, int32_t* status,
                                         void* stream) {
  CommitArgs a;
  const int rc = commit_args(p_max, top_id, tau, k_new, v_new, k_cache, v_cache, block_table,
                             cache_len, n_accepted, accepted_ids, commit_pos, n_layers, S, B,
                             n_kv_heads, head_dim, page_size, max_pages, num_pages, dtype, status,
                             &a);
  if (rc != MARS_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(accept_decide_kernel, dim3((S + 3) / 4), dim3(256), 0, st, a);
  const dim3 grid(S, n_layers);
  if (dtype == MARS_BF16)
    hipLaunchKernelGGL(commit_layers_kernel<2>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(commit_layers_kernel<4>, grid, dim3(256), 0, st, a);
  return mars_launch_status();
}

extern "C" const char* mars_strerror(int code) {
  switch (code) {
    case MARS_OK: return "ok";
    case MARS_ERR_NULL: return "a required pointer is NULL";
    case MARS_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case MARS_ERR_DTYPE: return "unknown dtype code";
    case MARS_ERR_UNSUPPORTED: return "valid but unsupported configuration";
    case MARS_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case MARS_ERR_WORKSPACE: return "workspace missing or too small";
    case MARS_ERR_LAUNCH: return "HIP launch error";
    default: return "unknown error code";
  }
}

extern "C" int mars_version(void) { return 100; }

namespace {
// Common path of the plain append and the gated block freeze.
int run_append(const void* k_rows, const void* v_rows, void* k_cache, void* v_cache,
               const int32_t* block_table, int32_t* cache_len, const int32_t* gate,
               int32_t gate_full, int32_t src_rows, int32_t S, int32_t T, int32_t n_kv_heads,
               int32_t head_dim, int32_t page_size, int32_t max_pages, int32_t num_pages,
               int32_t dtype, int32_t* status, void* stream) {
  MARS_REQUIRE(k_rows && v_rows && k_cache && v_cache && block_table && cache_len,
               MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_F32 || dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(S >= 1 && S <= 65535 && T >= 1 && T <= (1 << 30), MARS_ERR_SHAPE);
  MARS_REQUIRE(src_rows >= T && src_rows <= (1 << 30), MARS_ERR_SHAPE);
  MARS_REQUIRE(n_kv_heads >= 1 && head_dim >= 8 && head_dim % 8 == 0, MARS_ERR_SHAPE);
  MARS_REQUIRE(page_size >= 1 && max_pages >= 1 && num_pages >= 1, MARS_ERR_SHAPE);
  MARS_REQUIRE((long long)max_pages * page_size <= (1LL << 30), MARS_ERR_SHAPE);
  MARS_REQUIRE(n_kv_heads <= 65535, MARS_ERR_SHAPE);
  MARS_REQUIRE(head_dim * (dtype == MARS_BF16 ? 2 : 4) <= kAppendMaxRowBytes,
               MARS_ERR_UNSUPPORTED);
  MARS_REQUIRE(mars_aligned16(k_rows) && mars_aligned16(v_rows) && mars_aligned16(k_cache) &&
                   mars_aligned16(v_cache) && mars_aligned16(block_table) &&
                   mars_aligned16(cache_len) && mars_aligned16(gate),
               MARS_ERR_ALIGN);
  AppendArgs a;
  a.k_rows = (const char*)k_rows;
  a.v_rows = (const char*)v_rows;
  a.k_cache = (char*)k_cache;
  a.v_cache = (char*)v_cache;
  a.block_table = block_table;
  a.cache_len = cache_len;
  a.status = status;
  a.gate = gate;
  a.gate_full = gate_full;
  a.src_rows = src_rows;
  a.S = S;
  a.T = T;
  a.Hkv = n_kv_heads;
  a.D = head_dim;
  a.page_size = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  hipStream_t st = (hipStream_t)stream;
  const long long nwg = (long long)((T + 7 + 63) / 64) * n_kv_heads;
  MARS_REQUIRE(nwg <= 2147483647LL, MARS_ERR_SHAPE);
  const dim3 grid((unsigned)nwg, S);
  const size_t lds = 64 * ((size_t)head_dim * (dtype == MARS_BF16 ? 2 : 4) + 4);
  if (dtype == MARS_BF16)
    hipLaunchKernelGGL(kv_append_kernel<2>, grid, dim3(256), lds, st, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<4>, grid, dim3(256), lds, st, a);
  hipLaunchKernelGGL(kv_append_len_kernel, dim3((S + 255) / 256), dim3(256), 0, st, a);
  return mars_launch_status();
}
}  // namespace

extern "C" int mars_kv_append(const void* k_rows, const void* v_rows, void* k_cache,
                              void* v_cache, const int32_t* block_table, int32_t* cache_len,
                              int32_t S, int32_t T, int32_t n_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t max_pages, int32_t num_pages,
                              int32_t dtype, int32_t* status, void* stream) {
  return run_append(k_rows, v_rows, k_cache, v_cache, block_table, cache_len, nullptr, 0, T, S,
                    T, n_kv_heads, head_dim, page_size, max_pages, num_pages, dtype, status,
                    stream);
}

extern "C" int mars_block_freeze(const void* k_rows, const void* v_rows, void* k_cache,
                                 void* v_cache, const int32_t* block_table, int32_t* cache_len,
                                 const int32_t* unfrozen, int32_t S, int32_t R, int32_t B_cache,
                                 int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                 int32_t max_pages, int32_t num_pages, int32_t dtype,
                                 int32_t* status, void* stream) {
  MARS_REQUIRE(unfrozen, MARS_ERR_NULL);
  MARS_REQUIRE(B_cache >= 1 && B_cache <= R, MARS_ERR_SHAPE);
  return run_append(k_rows, v_rows, k_cache, v_cache, block_table, cache_len, unfrozen, B_cache,
                    R, S, B_cache, n_kv_heads, head_dim, page_size, max_pages, num_pages, dtype,
                    status, stream);
}

// ------------------------------------------------ batch-synchronous accept ----
namespace {

struct SyncArgs {
  const float* p_max;
  const int32_t* top_id;
  const float* tau;
  int32_t* unfrozen;
  int32_t* block_tokens;
  int32_t* n_kept;
  int32_t* n_rows;
  int32_t* status;
  int S, B, B_cache, policy;
};

// One workgroup for the whole batch: the block either froze for every
// sequence or for none, and policy 0 needs the batch minimum of the accepted
// counts, so the step is one block-wide decision.
__global__ __launch_bounds__(1024) void block_sync_accept_kernel(SyncArgs p) {
  __shared__ int wave_min[16];
  const int tid = threadIdx.x;
  int full = 1, nmin = 0x7FFFFFFF, bad = 0;
  for (int s = tid; s < p.S; s += 1024) {
    const int u = p.unfrozen[s];
    bad |= u < 0 || u > p.B_cache;
    full &= u == p.B_cache;
    nmin = min(nmin, accepted_count(p.p_max + (size_t)s * p.B, p.B, p.tau[s]));
  }
  if (__syncthreads_or(bad) && tid == 0) status_or(p.status, MARS_STATUS_CACHE_OVERFLOW);
  // the forward of this step froze the block iff every block was full
  const bool froze = __syncthreads_and(full) != 0;
  for (int o = 32; o > 0; o >>= 1) nmin = min(nmin, __shfl_xor(nmin, o));
  if ((tid & 63) == 0) wave_min[tid >> 6] = nmin;
  __syncthreads();
  nmin = wave_min[0];
  for (int w = 1; w < 16; ++w) nmin = min(nmin, wave_min[w]);
  for (int s = tid; s < p.S; s += 1024) {
    int32_t* toks = p.block_tokens + (size_t)s * p.B_cache;
    int u = min(max(p.unfrozen[s], 0), p.B_cache);
    if (froze) {
      u = 0;
      for (int i = 0; i < p.B_cache; ++i) toks[i] = -1;
    }
    const int n = p.policy == 0 ? nmin
                                : accepted_count(p.p_max + (size_t)s * p.B, p.B, p.tau[s]);
    const int keep = min(n, p.B_cache - u);
    for (int i = 0; i < keep; ++i) toks[u + i] = p.top_id[(size_t)s * p.B + i];
    p.unfrozen[s] = u + keep;
    p.n_kept[s] = keep;
    p.n_rows[s] = u + keep + p.B;
  }
}

}  // namespace

extern "C" int mars_block_sync_accept(const float* p_max, const int32_t* top_id,
                                      const float* tau, int32_t* unfrozen,
                                      int32_t* block_tokens, int32_t* n_kept, int32_t* n_rows,
                                      int32_t S, int32_t B, int32_t B_cache, int32_t policy,
                                      int32_t* status, void* stream) {
  MARS_REQUIRE(p_max && top_id && tau && unfrozen && block_tokens && n_kept && n_rows,
               MARS_ERR_NULL);
  MARS_REQUIRE(S >= 1 && S <= (1 << 24) && B >= 1 && B <= kMaxB, MARS_ERR_SHAPE);
  MARS_REQUIRE(B_cache >= 1 && B_cache <= 4096, MARS_ERR_SHAPE);
  MARS_REQUIRE(policy == 0 || policy == 1, MARS_ERR_SHAPE);
  SyncArgs a;
  a.p_max = p_max;
  a.top_id = top_id;
  a.tau = tau;
  a.unfrozen = unfrozen;
  a.block_tokens = block_tokens;
  a.n_kept = n_kept;
  a.n_rows = n_rows;
  a.status = status;
  a.S = S;
  a.B = B;
  a.B_cache = B_cache;
  a.policy = policy;
  hipLaunchKernelGGL(block_sync_accept_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, a);
  return mars_launch_status();
}
