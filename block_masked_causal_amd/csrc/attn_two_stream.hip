// Two-stream MARS attention forward (training form) for gfx950.
//
// The mask is the 2L x 2L matrix M of the papernotes.org notes on "MARS:
// Enabling Autoregressive Models Multi-Token Generation", key design 1
// (关键设计 1), equation M_ij, over z = [x; x~] with beta(t) = ceil(t/B).
// It is never materialised: every query row a owns at most two visible key
// intervals, computed once per row in registers,
//     clean row a < L : [0, a]
//     mask row a >= L : [0, b*B) and [L + b*B, a]      (t = a - L, b = t / B)
// and a key c is visible iff it lies in one of them. Whole key tiles outside
// a query tile's intervals are never loaded, and tiles entirely inside them
// skip the per-element test.
#include "mars_common.hpp"

using namespace mars;

namespace {

struct TwoStreamArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int batch, L, B, Hq, Hkv, twoL, group;
  float scale_log2;  // softmax_scale * log2(e): scores are kept in log2 units
  int mask_mode;     // 0 = MARS two-stream mask, 1 = causal over all 2L
  int nqt;           // query tiles per (batch, head)
};

// Visible keys of row a: c < hi1, or lo2 <= c < hi2.
__device__ __forceinline__ void row_intervals(int a, int L, int B, int mode, int& hi1, int& lo2,
                                              int& hi2) {
  if (mode == 1 || a < L) {
    hi1 = a + 1;
    lo2 = 0;
    hi2 = 0;
    return;
  }
  const int bb = ((a - L) / B) * B;
  hi1 = bb;
  lo2 = L + bb;
  hi2 = a + 1;
}

__device__ __forceinline__ bool in_rows(int c, int hi1, int lo2, int hi2) {
  return (c < hi1) | ((c >= lo2) & (c < hi2));
}

// ---------------------------------------------------------------------------
// float32 path: one wave per 64 query rows, K/V staged in LDS 32 keys at a
// time, one query row per lane. Used for the small fp32 configuration.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void two_stream_f32_kernel(TwoStreamArgs p) {
  constexpr int KT = 32;
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];
  const int lane = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int a = blockIdx.x * 64 + lane;
  const int kvh = h / p.group;
  const bool valid = a < p.twoL;
  const float* Q = (const float*)p.q;
  const float* K = (const float*)p.k;
  const float* V = (const float*)p.v;
  const size_t qrow = ((size_t)b * p.twoL + (valid ? a : 0)) * p.Hq + h;

  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? Q[qrow * D + d] * p.scale_log2 : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  int hi1, lo2, hi2;
  row_intervals(a, p.L, p.B, p.mask_mode, hi1, lo2, hi2);
  const int a_last = min((int)blockIdx.x * 64 + 63, p.twoL - 1);
  for (int c0 = 0; c0 <= a_last; c0 += KT) {
    __syncthreads();
    for (int idx = lane; idx < KT * D; idx += 64) {
      const int c = c0 + idx / D, d = idx % D;
      const size_t kr = ((size_t)b * p.twoL + c) * p.Hkv + kvh;
      Ks[idx / D][d] = c < p.twoL ? K[kr * D + d] : 0.f;
      Vs[idx / D][d] = c < p.twoL ? V[kr * D + d] : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < KT; ++jj) {
      const int c = c0 + jj;
      if (!valid || c >= p.twoL || !in_rows(c, hi1, lo2, hi2)) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], Ks[jj][d], s);
      const float mn = fmaxf(m, s);
      const float alpha = exp2f(m - mn);
      const float pe = exp2f(s - mn);
      l = l * alpha + pe;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], alpha, pe * Vs[jj][d]);
      m = mn;
    }
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* O = (float*)p.o;
#pragma unroll
  for (int d = 0; d < D; ++d) O[qrow * D + d] = o[d] * inv;
  if (p.lse) p.lse[((size_t)b * p.Hq + h) * p.twoL + a] = (m + log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// bfloat16 MFMA path.
//
// Workgroup = 4 waves = 128 query rows of one (batch, q-head); each wave owns
// 32 rows. Scores are computed transposed, S^T = K Q^T, with the 32x32x16
// MFMA: lane (j = l % 32, hf = l / 32) then holds query row j and 16 of the
// keys of each 32-key sub-tile, so the row softmax needs one cross-lane
// exchange (lane l <-> l ^ 32). The probabilities stay in registers and feed
// O^T = V^T P^T directly as the B operand: K slot (hf, e) of a 16-key chunk
// is mapped to key 4*hf + e (e < 4) or 8 + 4*hf + e - 4 (e >= 4), exactly the
// keys the lane already holds. V is written to LDS transposed ([d][key]) so
// that the A operand is two 8-byte LDS reads.
// ---------------------------------------------------------------------------
template <int D>
struct Cfg {
  static constexpr int BM = 128;      // query rows per workgroup
  static constexpr int BN = 64;       // keys per tile
  static constexpr int KST = D + 8;   // K tile row stride in LDS (elements)
  static constexpr int VST = BN + 4;  // V^T tile row stride in LDS (elements)
  static constexpr int KSZ = BN * KST;
  static constexpr int VSZ = D * VST;
  static constexpr int KLOADS = BN * D / 8 / 256;             // 16-byte K loads per thread
  static constexpr int VPATCH = (BN / 4) * (D / 8);           // 4-key x 8-dim V patches
  static constexpr int VLOADS = (VPATCH + 255) / 256;         // patches per thread
  static constexpr size_t LDS_BYTES = 2 * (KSZ + VSZ) * sizeof(bf16_t);
};

template <int D>
__global__ __launch_bounds__(256, 2) void two_stream_bf16_kernel(TwoStreamArgs p) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;

  // ---- which (batch, head, query tile): heaviest query tiles first --------
  const int bh_count = p.batch * p.Hq;
  const int bh = blockIdx.x % bh_count;
  const int rank = blockIdx.x / bh_count;
  const int b = bh / p.Hq, h = bh % p.Hq;
  int qt;
  if (p.mask_mode == 0 && (p.L % C::BM) == 0) {
    const int nqs = p.L / C::BM;  // tiles per stream; clean tile i and mask tile i cost alike
    qt = (rank & 1) * nqs + (nqs - 1 - (rank >> 1));
  } else {
    qt = p.nqt - 1 - rank;
  }
  const int a0 = qt * C::BM;
  const int a_last = min(a0 + C::BM, p.twoL) - 1;
  const int kvh = h / p.group;

  // ---- key ranges this query tile needs, and which tiles are fully visible
  int r1_hi, r2_lo = 0, r2_hi = 0, full_below;
  if (p.mask_mode == 1 || a_last < p.L) {
    r1_hi = a_last + 1;
    full_below = a0 + 1;  // a tile is fully visible iff its last key <= a0
  } else if (a0 >= p.L) {
    const int t0 = a0 - p.L, t1 = a_last - p.L;
    const int b0B = (t0 / p.B) * p.B, b1B = (t1 / p.B) * p.B;
    r1_hi = b1B;          // clean keys of strictly earlier blocks
    full_below = b0B;
    r2_lo = p.L + b0B;    // mask keys of the blocks in this tile
    r2_hi = a_last + 1;
  } else {
    r1_hi = a_last + 1;   // tile straddles the stream boundary: test every key
    full_below = 0;
  }
  const int n1 = (r1_hi + C::BN - 1) / C::BN;
  const int n2 = r2_hi > r2_lo ? (r2_hi - r2_lo + C::BN - 1) / C::BN : 0;
  const int ntiles = n1 + n2;

  // ---- this lane's query row ----------------------------------------------
  const int a = a0 + w * 32 + j;
  int hi1, lo2, hi2;
  row_intervals(a, p.L, p.B, p.mask_mode, hi1, lo2, hi2);
  const bf16_t* Qg = (const bf16_t*)p.q;
  bf16x8 qf[D / 16];
  if (a < p.twoL) {
    const bf16_t* qrow = Qg + (((size_t)b * p.twoL + a) * p.Hq + h) * D + 8 * hf;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qf[c] = *(const bf16x8*)(qrow + 16 * c);
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qf[c] = bf16x8{};
  }

  const size_t rs = (size_t)p.Hkv * D;  // element stride between consecutive keys
  const bf16_t* Kg = (const bf16_t*)p.k + (size_t)b * p.twoL * rs + (size_t)kvh * D;
  const bf16_t* Vg = (const bf16_t*)p.v + (size_t)b * p.twoL * rs + (size_t)kvh * D;

  u32x4 kreg[C::KLOADS];
  u32x4 vreg[C::VLOADS][4];

  auto tile_c0 = [&](int it) { return it < n1 ? it * C::BN : r2_lo + (it - n1) * C::BN; };

  auto load_tile = [&](int it) {
    const int c0 = tile_c0(it);
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      const int c = c0 + row;
      kreg[i] = c < p.twoL ? *(const u32x4*)(Kg + c * rs + ch * 8) : u32x4{};
    }
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) {
      const int pi = tid + 256 * i;
      const int dg = pi % (D / 8), kg = pi / (D / 8);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int c = c0 + 4 * kg + rr;
        vreg[i][rr] = (pi < C::VPATCH && c < p.twoL) ? *(const u32x4*)(Vg + c * rs + dg * 8)
                                                      : u32x4{};
      }
    }
  };

  auto store_tile = [&](int buf) {
    bf16_t* Ks = lds + buf * (C::KSZ + C::VSZ);
    bf16_t* Vt = Ks + C::KSZ;
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      *(u32x4*)(Ks + row * C::KST + ch * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) {
      const int pi = tid + 256 * i;
      if (pi >= C::VPATCH) continue;
      const int dg = pi % (D / 8), kg = pi / (D / 8);
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        const uint32_t x0 = vreg[i][0][dw], x1 = vreg[i][1][dw];
        const uint32_t x2 = vreg[i][2][dw], x3 = vreg[i][3][dw];
        // dimension 8*dg + 2*dw: low halves; dimension 8*dg + 2*dw + 1: high halves
        u32x2 lo = {(x0 & 0xFFFFu) | (x1 << 16), (x2 & 0xFFFFu) | (x3 << 16)};
        u32x2 hi = {(x0 >> 16) | (x1 & 0xFFFF0000u), (x2 >> 16) | (x3 & 0xFFFF0000u)};
        *(u32x2*)(Vt + (8 * dg + 2 * dw) * C::VST + 4 * kg) = lo;
        *(u32x2*)(Vt + (8 * dg + 2 * dw + 1) * C::VST + 4 * kg) = hi;
      }
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) load_tile(it + 1);

    const bf16_t* Ks = lds + (it & 1) * (C::KSZ + C::VSZ);
    const bf16_t* Vt = Ks + C::KSZ;
    const int c0 = tile_c0(it);
    const bool in_r1 = it < n1;
    const int lim_lo = in_r1 ? 0 : r2_lo;
    const int lim_hi = in_r1 ? r1_hi : r2_hi;
    const bool partial = !(in_r1 && c0 + C::BN - 1 < full_below);

    // S^T for two 32-key sub-tiles
    f32x16 s[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      s[n] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 ka = *(const bf16x8*)(Ks + (32 * n + j) * C::KST + 16 * c + 8 * hf);
        s[n] = mfma32(ka, qf[c], s[n]);
      }
    }

    float mt = -INFINITY;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[n][r] * p.scale_log2;
        if (partial) {
          const int c = c0 + 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3);
          const bool vis = (c >= lim_lo) & (c < lim_hi) & in_rows(c, hi1, lo2, hi2);
          x = vis ? x : -INFINITY;
        }
        s[n][r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m, mt);
    const float mb = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - mb);
    float rsum = 0.f;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(s[n][r] - mb);
        s[n][r] = e;
        rsum += e;
      }
    }
    l = l * alpha + rsum;
    m = mnew;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] *= alpha;

    bf16x8 pb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[kc][e] = (bf16_t)s[kc >> 1][8 * (kc & 1) + e];
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16_t* vr = Vt + (32 * i + j) * C::VST + 16 * kc + 4 * hf;
        const bf16x4 vlo = *(const bf16x4*)vr;
        const bf16x4 vhi = *(const bf16x4*)(vr + 8);
        const bf16x8 va = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
        o[i] = mfma32(va, pb[kc], o[i]);
      }
    }

    if (it + 1 < ntiles) store_tile((it + 1) & 1);
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32);
  if (a >= p.twoL) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  bf16_t* orow = (bf16_t*)p.o + (((size_t)b * p.twoL + a) * p.Hq + h) * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk = {pack_bf16x2(o[i][4 * g] * inv, o[i][4 * g + 1] * inv),
                  pack_bf16x2(o[i][4 * g + 2] * inv, o[i][4 * g + 3] * inv)};
      *(u32x2*)(orow + 32 * i + 8 * g + 4 * hf) = pk;
    }
  }
  if (p.lse && hf == 0) p.lse[((size_t)b * p.Hq + h) * p.twoL + a] = (m + log2f(lt)) * kLn2;
}

template <int D>
int launch_bf16(const TwoStreamArgs& a, hipStream_t st) {
  using C = Cfg<D>;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)two_stream_bf16_kernel<D>,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)C::LDS_BYTES) != hipSuccess)
      return MARS_ERR_LAUNCH;
    attr_set = true;
  }
  const int nblocks = a.batch * a.Hq * a.nqt;
  hipLaunchKernelGGL(two_stream_bf16_kernel<D>, dim3(nblocks), dim3(256), C::LDS_BYTES, st, a);
  return mars_launch_status();
}

template <int D>
int launch_f32(const TwoStreamArgs& a, hipStream_t st) {
  dim3 grid((a.twoL + 63) / 64, a.Hq, a.batch);
  hipLaunchKernelGGL(two_stream_f32_kernel<D>, grid, dim3(64), 0, st, a);
  return mars_launch_status();
}

}  // namespace

extern "C" int mars_attn_two_stream(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int32_t batch, int32_t L, int32_t B,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t dtype, float softmax_scale, int32_t mask_mode,
                                    void* stream) {
  MARS_REQUIRE(q && k && v && o, MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_F32 || dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(batch >= 1 && L >= 1 && B >= 1 && B <= L && L <= (1 << 29), MARS_ERR_SHAPE);
  MARS_REQUIRE(n_q_heads >= 1 && n_kv_heads >= 1 && n_q_heads % n_kv_heads == 0, MARS_ERR_SHAPE);
  MARS_REQUIRE(mask_mode == 0 || mask_mode == 1, MARS_ERR_SHAPE);
  MARS_REQUIRE(head_dim >= 1, MARS_ERR_SHAPE);
  MARS_REQUIRE(mars_aligned16(q) && mars_aligned16(k) && mars_aligned16(v) &&
                   mars_aligned16(o) && mars_aligned16(lse),
               MARS_ERR_ALIGN);
  const int twoL = 2 * L;
  // Element offsets must fit the kernels' index arithmetic.
  MARS_REQUIRE((double)batch * twoL * n_q_heads * head_dim < 9.0e18, MARS_ERR_SHAPE);
  MARS_REQUIRE((double)twoL * n_kv_heads * head_dim < 2147483647.0, MARS_ERR_SHAPE);

  TwoStreamArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.batch = batch;
  a.L = L;
  a.B = B;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.twoL = twoL;
  a.group = n_q_heads / n_kv_heads;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  a.scale_log2 = scale * kLog2e;
  a.mask_mode = mask_mode;
  hipStream_t st = (hipStream_t)stream;

  if (dtype == MARS_BF16) {
    a.nqt = (twoL + Cfg<64>::BM - 1) / Cfg<64>::BM;
    MARS_REQUIRE((double)batch * n_q_heads * a.nqt < 2147483647.0, MARS_ERR_SHAPE);
    if (head_dim == 64) return launch_bf16<64>(a, st);
    if (head_dim == 128) return launch_bf16<128>(a, st);
    return MARS_ERR_UNSUPPORTED;
  }
  a.nqt = (twoL + 63) / 64;
  MARS_REQUIRE(n_q_heads <= 65535 && batch <= 65535, MARS_ERR_SHAPE);
  if (head_dim == 32) return launch_f32<32>(a, st);
  if (head_dim == 64) return launch_f32<64>(a, st);
  if (head_dim == 128) return launch_f32<128>(a, st);
  return MARS_ERR_UNSUPPORTED;
}
