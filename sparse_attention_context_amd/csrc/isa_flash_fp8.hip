// FP8 (e4m3) variant of the ISA full route on gfx950 MX-scaled MFMA.
//
// The first page's list of attention speed-ups names 8-bit quantisation;
// this variant computes the full route of "Lightning Unified Video Editing
// via In-Context Sparse Attention" (exact softmax attention over the tokens
// of the kept key set) with its operands in OCP e4m3 under power-of-two
// block scales (MX: one shared 2^e per 32 elements, e the smallest with
// max|x| / 2^e <= 448):
//   Q per (query row, 32 d), K per (key row, 32 d), V per (d, 32 keys of the
//   key list from its start), P = exp2(x - m) unscaled, m the reference
//   maximum kept at a whole number in the exp2 domain (so P rounds as
//   P_exact * 2^k does).
// v_mfma_scale_f32_32x32x64_f8f6f4 (measured on the GPU): lane l holds row
// (A) / column (B) l%32; byte t of lane half h is k = 32 (t/16) + 16 h + t%16;
// the e8m0 scale of row i and k-block b (32 consecutive k) comes from lane
// i + 32 b; the accumulator has the usual 32x32 layout; 64 cycles per
// instruction (twice the bf16 rate).
//
// pack: the full route's key list (source rows, then the tokens of the kept
//   context blocks) in e4m3: K8 [BH][nkp][D] with scales [BH][nkp][D/32], and
//   per 64-key tile V8T [BH][tile][D][64] with scales [BH][tile][D][2].  Row d
//   of a V8T tile holds, at byte 32 h + t, key 32 (t/16) + 8 ((t%16)/4) + 4 h
//   + t%4: the order in which a lane of S^T = K Q^T holds its keys, so the
//   probabilities are the B operand of O^T += V^T P^T with no shuffle, and the
//   MX blocks of that product are the two 32-key halves of the tile.
// flash: 8 waves x 32 query rows, 64-key tiles, 2-stage LDS ring; Q quantised
//   at load; otherwise the structure of the bf16 kernel (lazy reference max,
//   split-K partials merged by the bf16 merge kernel).
#include "isa_device.h"
#include "isa_kernels.h"
#include "isa_split.h"

namespace isa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

// two 16-byte LDS reads as one 8-register MFMA operand
__device__ __forceinline__ v8i lds_operand(const char* lo, const char* hi) {
  const v4i a = *(const v4i*)lo;
  const v4i b = *(const v4i*)hi;
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Smallest e with amax / 2^e <= 448, from the float's bits (exact); e8m0
// range.  448 = 1.75 * 2^8: amax = 1.f * 2^(E-127) fits 2^(E-135) * 448 when
// 1.f <= 1.75.
__device__ __forceinline__ int block_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int E = (int)(u >> 23);
  if (E == 0) return -127;
  const int e = E - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return max(-127, min(127, e));
}

// 2^-e as a float (|e| <= 127 and -e >= -126 for the values used here).
__device__ __forceinline__ float pow2_neg(int e) {
  const int b = 127 - e;
  return b >= 1 ? __uint_as_float((uint32_t)b << 23) : 0.0f;
}

// four floats -> four e4m3 bytes (round to nearest even)
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int v = 0;
  v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, v, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

struct Fp8Args {
  const void* Q;
  void* O;
  const void* K;
  const void* V;
  RowMap rmq, rmo, rmk, rmv;   // element strides of Q, O, K, V
  const int* ctx_rows;   // [BH][ctx_tok]
  const int* kept;       // [BH][kc]
  long long ctx_tok;
  int kc, nb_c, b, tail_c;
  uint8_t* k8;           // [BH][nkp][D]
  uint8_t* ks;           // [BH][nkp][D/32]
  uint8_t* v8t;          // [BH][ntile][D][64]
  uint8_t* vs;           // [BH][ntile][D][2]
  int nkp, ntile;
  const int* q_list;
  int q_k, nb_s;
  float* lse;
  bf16_t* part_o;
  float* part_ml;
  int nsplit, tiles_per_split;
  int Ns, Nk;
  int row_tiles;
  int n_wg;
  float scale_log2;      // log2(e)/sqrt(d)
  // d = 128: the stream-K split of the bf16 full route (isa_split.h)
  long long sk_U;
  int sk_G, sk_P, sk_T, sk_R0, sk_K, sk_grid, sk_q, sk_x;
};

// ---------------------------------------------------------------------------
// pack: one workgroup per (64-key tile, head)

template <int D>
__global__ __launch_bounds__(256) void isa_fp8_pack_kernel(Fp8Args a) {
  constexpr int BN = 64, NB = D / 32;
  __shared__ float vt[BN][D + 1];
  const int tile = blockIdx.x;
  const long long bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int n_keys = a.Ns + (int)a.ctx_tok;
  auto key_row = [&](int t) -> int {
    if (t < a.Ns) return t;
    if (t < n_keys) return a.ctx_rows[bh * a.ctx_tok + (t - a.Ns)];
    return -1;
  };
  // K rows: one thread per (key, 32-d block)
  if (tid < BN * NB) {
    const int i = tid / NB, kb = tid % NB;
    const int t = tile * BN + i;
    const int row = key_row(t);
    float x[32];
    if (row >= 0) {
      const bf16_t* kp = (const bf16_t*)a.K + rm_head(a.rmk, bh) + (long long)row * a.rmk.sn + kb * 32;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 w = *(const u32x4*)(kp + 8 * c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[8 * c + 2 * j] = __uint_as_float(w[j] << 16);
          x[8 * c + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) x[j] = 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(x[j]));
    const int e = m > 0.f ? block_exp(m) : 0;
    const float s = pow2_neg(e);
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = pack4_fp8(x[4 * j] * s, x[4 * j + 1] * s, x[4 * j + 2] * s, x[4 * j + 3] * s);
    uint8_t* dst = a.k8 + (bh * a.nkp + t) * D + kb * 32;
    *(u32x4*)dst = u32x4{out[0], out[1], out[2], out[3]};
    *(u32x4*)(dst + 16) = u32x4{out[4], out[5], out[6], out[7]};
    a.ks[(bh * a.nkp + t) * NB + kb] = (uint8_t)(e + 127);
  }
  // V tile into LDS (fp32), zero rows past the list
  for (int q = tid; q < BN * (D / 8); q += 256) {
    const int i = q / (D / 8), c = q % (D / 8);
    const int row = key_row(tile * BN + i);
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (row >= 0) w = *(const u32x4*)((const bf16_t*)a.V + rm_head(a.rmv, bh) + (long long)row * a.rmv.sn + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vt[i][c * 8 + 2 * j] = __uint_as_float(w[j] << 16);
      vt[i][c * 8 + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  __syncthreads();
  // V^T rows: one thread per (d, 32-key half hb)
  for (int q = tid; q < D * 2; q += 256) {
    const int d = q >> 1, hb = q & 1;
    float m = 0.f;
    for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(vt[32 * hb + j][d]));
    const int e = m > 0.f ? block_exp(m) : 0;
    const float s = pow2_neg(e);
    uint8_t* dst = a.v8t + ((bh * a.ntile + tile) * D + d) * 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // bytes 32 h + 16 hb + j hold key 32 hb + 8 (j/4) + 4 h + j%4
      uint32_t w[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int k0 = 32 * hb + 8 * g + 4 * h;
        w[g] = pack4_fp8(vt[k0][d] * s, vt[k0 + 1][d] * s, vt[k0 + 2][d] * s, vt[k0 + 3][d] * s);
      }
      *(u32x4*)(dst + 32 * h + 16 * hb) = u32x4{w[0], w[1], w[2], w[3]};
    }
    a.vs[((bh * a.ntile + tile) * D + d) * 2 + hb] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------
// flash (full route)

template <int D>
__global__ __launch_bounds__(512) void isa_flash_fp8_kernel(Fp8Args a) {
  constexpr int NW = 8, NTHR = NW * 64, BN = 64, BM = 32 * NW, NB = D / 32, NU = D / 64;
  constexpr int KRS = D + 16, VRS = 64 + 16;
  constexpr int KT = BN * KRS, VT = D * VRS;
  constexpr int OFF_V = KT, OFF_KS = KT + VT, OFF_VS = OFF_KS + BN * 4;
  constexpr int STAGE = OFF_VS + D * 2;
  constexpr int NT = D / 32;
  static_assert(BN * D / 16 <= NTHR, "one 16-byte chunk of K8 and of V8T per thread");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  // work item lid: row tile fastest, then key split, then head (as the
  // forward flash kernels), so that the workgroups running at once on an XCD
  // share one K/V range in its L2
  const int lid = xcd_remap(blockIdx.x, a.n_wg);
  const int rt = lid % a.row_tiles;
  const int rest = lid / a.row_tiles;
  const int split = rest % a.nsplit;
  const int bh = rest / a.nsplit;

  // ---- query row, quantised: byte t of lane half h in MFMA u is d = 64u + 32(t/16) + 16h + t%16
  const long long vrow = (long long)rt * BM + w * 32 + l32;
  const int qrow = route_row(a.q_list + (long long)bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
  v8i qB[NU];
  int qS[NU];
  {
    const bf16_t* qp = (const bf16_t*)a.Q + rm_head(a.rmq, bh) + (long long)(qrow < 0 ? 0 : qrow) * a.rmq.sn;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float x[32];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16_t* p = qp + 64 * u + 32 * b + 16 * h;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 wv = *(const u32x4*)(p + 8 * c);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[16 * b + 8 * c + 2 * j] = __uint_as_float(wv[j] << 16);
            x[16 * b + 8 * c + 2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
          }
        }
      }
      // block b of this MFMA is d in [64u + 32b, +32): 16 values here, 16 in lane half 1-h
      int eb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(x[16 * b + j]));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        eb[b] = m > 0.f ? block_exp(m) : 0;
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float s = pow2_neg(eb[g >> 2]);
        qB[u][g] = (int)pack4_fp8(x[4 * g] * s, x[4 * g + 1] * s, x[4 * g + 2] * s, x[4 * g + 3] * s);
      }
      qS[u] = eb[h] + 127;  // this lane supplies the scale of block h
    }
  }

  // ---- key range
  const int n_keys = a.Ns + (int)a.ctx_tok;
  const bool tail_kept = a.kc > 0 && a.kept[(long long)bh * a.kc + a.kc - 1] == a.nb_c - 1;
  const int n_valid = n_keys - (tail_kept ? a.b - a.tail_c : 0);
  const int ntiles = (n_keys + BN - 1) / BN;
  const int t_begin = split * a.tiles_per_split;
  const int nt = max(0, min(a.tiles_per_split, ntiles - t_begin));
  const int t_last = t_begin + nt - 1;

  const uint8_t* Kg = a.k8 + (long long)bh * a.nkp * D;
  const uint8_t* KSg = a.ks + (long long)bh * a.nkp * NB;
  const uint8_t* Vg = a.v8t + (long long)bh * a.ntile * D * 64;
  const uint8_t* VSg = a.vs + (long long)bh * a.ntile * D * 2;

  // per tile: K8 64 x D bytes and V8T D x 64 bytes (D/16*4 16-byte chunks
  // each), key scales 64 x NB bytes, value scales D x 2 bytes
  constexpr int KCH = BN * D / 16, NKC = (KCH + NTHR - 1) / NTHR;
  struct Staged { u32x4 k[NKC]; u32x4 v[NKC]; uint32_t ks, vs; };
  auto load = [&](int tile) -> Staged {
    Staged g;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int q = tid + NTHR * i;
      g.k[i] = u32x4{0u, 0u, 0u, 0u};
      g.v[i] = u32x4{0u, 0u, 0u, 0u};
      if (q < KCH) {
        g.k[i] = *(const u32x4*)(Kg + (long long)tile * BN * D + q * 16);
        g.v[i] = *(const u32x4*)(Vg + (long long)tile * D * 64 + q * 16);
      }
    }
    g.ks = 0u;
    g.vs = 0u;
    if (tid < BN) {
      uint32_t v = 0u;
#pragma unroll
      for (int b = 0; b < NB; ++b) v |= (uint32_t)KSg[((long long)tile * BN + tid) * NB + b] << (8 * b);
      g.ks = v;
    }
    if (tid < D) g.vs = *(const uint16_t*)(VSg + ((long long)tile * D + tid) * 2);
    return g;
  };
  auto store = [&](int stage, const Staged& g) {
    char* S0 = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int q = tid + NTHR * i;
      if (q < KCH) {
        *(u32x4*)(S0 + (q / (D / 16)) * KRS + (q % (D / 16)) * 16) = g.k[i];
        *(u32x4*)(S0 + OFF_V + (q / 4) * VRS + (q % 4) * 16) = g.v[i];
      }
    }
    if (tid < BN) ((uint32_t*)(S0 + OFF_KS))[tid] = g.ks;
    if (tid < D) ((uint16_t*)(S0 + OFF_VS))[tid] = (uint16_t)g.vs;
  };

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;   // m_ref: exp2 domain, a whole number once set
  const float sc = a.scale_log2;

  auto tile_step = [&](int j, int stage) {
    const char* S0 = smem + stage * STAGE;
    const int t0 = (t_begin + j) * BN;
    f32x16 S[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      S[half] = f32x16{};
      const int krow = half * 32 + l32;
      const uint32_t ksw = ((const uint32_t*)(S0 + OFF_KS))[krow];
      const char* kp = S0 + krow * KRS + 16 * h;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const v8i ka = lds_operand(kp + 64 * u, kp + 64 * u + 32);
        const int kscale = (int)((ksw >> (8 * (2 * u + h))) & 0xffu);
        S[half] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qB[u], S[half], 0, 0, 0, kscale, 0, qS[u]);
      }
    }
    // softmax in the exp2 domain; keys past the range (a short kept tail) are masked
    // raw logits (the scale sc > 0 is applied in the exp2 argument)
    float x[32];
    float mx = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[16 * half + r] = S[half][r];
        mx = fmaxf(mx, x[16 * half + r]);
      }
    if (t0 + BN > n_valid) {  // only the last tile of the range can be partial
      mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int key = 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * h + (i & 3);
        if (t0 + key >= n_valid) x[i] = -INFINITY;
        mx = fmaxf(mx, x[i]);
      }
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 32)) * sc;
    const bool move = mx > m_ref + 8.0f;
    if (__ballot(move)) {
      const float m_new = move ? ceilf(mx) : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
      m_ref = m_new;
    }
    float psum = 0.f;
    v8i pB;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(x[4 * g + e], sc, -m_ref));
        psum += p[e];
      }
      pB[g] = (int)pack4_fp8(p[0], p[1], p[2], p[3]);
    }
    l_run += psum;
    // O^T += V^T P^T: lane (d, h) reads V8T row d bytes [32h, 32h+32); value scale of key half h
    const uint16_t* vsw = (const uint16_t*)(S0 + OFF_VS);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int d = 32 * t + l32;
      const char* vp = S0 + OFF_V + d * VRS + 32 * h;
      const v8i va = lds_operand(vp, vp + 16);
      const int vscale = (int)((vsw[d] >> (8 * h)) & 0xffu);
      acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pB, acc[t], 0, 0, 0, vscale, 0, 127);
    }
  };

  if (nt > 0) {
    store(0, load(t_begin));
    __syncthreads();
  }
  for (int j = 0; j < nt; ++j) {
    const Staged g = load(min(t_begin + j + 1, t_last));
    tile_step(j, j & 1);
    if (j + 1 < nt) store((j + 1) & 1, g);
    __syncthreads();
  }

  // ---- epilogue (the layout of the bf16 kernel; partials merged by its merge kernel)
  const float l_tot = l_run + wave_shfl_xor(l_run, 32);
  if (a.nsplit == 1) {
    if (qrow < 0) return;
    const float inv = 1.0f / l_tot;
    bf16_t* op = (bf16_t*)a.O + rm_head(a.rmo, bh) + (long long)qrow * a.rmo.sn;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(u32x2*)(op + 32 * t + 8 * g + 4 * h) =
            u32x2{pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv),
                  pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv)};
    if (a.lse && h == 0) a.lse[(long long)bh * a.Ns + qrow] = m_ref + __builtin_log2f(l_tot);
  } else {
    const long long prow = ((long long)bh * a.row_tiles * BM + vrow) * a.nsplit + split;
    bf16_t* po = a.part_o + prow * D;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(u32x2*)(po + 32 * t + 8 * g + 4 * h) =
            u32x2{pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv),
                  pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv)};
    // the merge expects the reference max in raw logit units
    if (h == 0) *(float2*)(a.part_ml + prow * 2) = float2{m_ref / sc, l_tot};
  }
}

// ---------------------------------------------------------------------------
// flash (full route), d = 128, on the ping-pong schedule of the bf16 token
// kernel (isa_flash.hip): two wave groups one barrier phase apart, each
// tile an MFMA phase X (O^T += V8^T P8^T of the previous tile, S = K8 Q8^T)
// and a VALU phase Y (softmax, probabilities to e4m3).  Here the softmax
// outweighs the 8 MX MFMAs of a tile, so the direct global->LDS loads of
// K8(j+3) and V8T(j+2) (tiles are contiguous after the pack) are issued at
// the end of X_j.  Four-stage rings: K(t) is issued in phases 2t-6 / 2t-5,
// after the last read of its stage (2t-7); V(t) in 2t-4 / 2t-3, after 2t-5;
// each wave waits for its loads of X_{j-1} before the barrier that closes
// Y_j, so K(t) has landed by 2t-2 (first read 2t) and V(t) by 2t (first
// read 2t+2).  Scales travel with their tiles.  LDS rows are unpadded and
// swizzled: K8 chunk c of row r at c ^ ((r >> 1) & 7), V8T chunk c of row d
// at c ^ ((d >> 2) & 3), which keeps the 16-byte operand reads on distinct
// banks.  Numerics are those of isa_flash_fp8_kernel.
__device__ __forceinline__ int k8_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int v8_swz(int d) { return (d >> 2) & 3; }

__global__ __launch_bounds__(512) void isa_flash_fp8_pp_kernel(Fp8Args a) {
  constexpr int D = 128, BN = 64, BM = 256, NB = D / 32, NU = D / 64, NT = D / 32, NST = 4;
  constexpr int KTB = BN * D, VTB = D * BN;   // K8 tile: 64 rows x 128 B; V8T tile: 128 rows x 64 B
  static_assert(BM == kFlashRows, "tile mapping");
  __shared__ __attribute__((aligned(1024))) char smem[NST * (KTB + VTB)];   // K8 ring, then V8T ring
  __shared__ __attribute__((aligned(256))) uint32_t sks[NST][BN];           // key scales, 4 per row
  __shared__ __attribute__((aligned(256))) uint32_t svs[NST][D / 2];        // value scales, 2 per d

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wg = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  // Work items: the items of stream-K workgroup g (the logical id; whole row
  // tiles, then the row tiles that its range meets), one after the other,
  // the pipeline drained between them.  Consecutive workgroups run on one XCD
  // and share its L2.
  const SkItems sk = sk_items(a, xcd_remap((int)blockIdx.x, (int)gridDim.x));
#pragma unroll 1
  for (int item = 0; item < sk.kdp + sk.nsk; ++item) {
    const SkItem it = sk_item(a, sk, item);
    const int bh = it.bh, rt = it.rt;
    const int part = it.part < 0 ? -1 : (it.part & 7), Rs = it.part >> 3;   // part < 0: the whole row tile
    if (item > 0) __syncthreads();   // the previous item's LDS reads are done

    // ---- query row, quantised as in isa_flash_fp8_kernel
    const long long vrow = (long long)rt * BM + w * 32 + l32;
    const int qrow = route_row(a.q_list + (long long)bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);
    v8i qB[NU];
    int qS[NU];
    {
      const bf16_t* qp = (const bf16_t*)a.Q + rm_head(a.rmq, bh) + (long long)(qrow < 0 ? 0 : qrow) * a.rmq.sn;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float x[32];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const bf16_t* p = qp + 64 * u + 32 * b + 16 * h;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const u32x4 wv = *(const u32x4*)(p + 8 * c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              x[16 * b + 8 * c + 2 * j] = __uint_as_float(wv[j] << 16);
              x[16 * b + 8 * c + 2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
            }
          }
        }
        int eb[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(x[16 * b + j]));
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          eb[b] = m > 0.f ? block_exp(m) : 0;
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const float sq = pow2_neg(eb[g >> 2]);
          qB[u][g] = (int)pack4_fp8(x[4 * g] * sq, x[4 * g + 1] * sq, x[4 * g + 2] * sq, x[4 * g + 3] * sq);
        }
        qS[u] = eb[h] + 127;
      }
    }

    // ---- key range
    const int n_keys = a.Ns + (int)a.ctx_tok;
    const bool tail_kept = a.kc > 0 && a.kept[(long long)bh * a.kc + a.kc - 1] == a.nb_c - 1;
    const int n_valid = n_keys - (tail_kept ? a.b - a.tail_c : 0);
    const int t_begin = it.t_begin;   // (rotated key order of a cut row tile: no wrap)
    const int nt = it.nt;

    const uint8_t* Kg = a.k8 + (long long)bh * a.nkp * D;
    const uint8_t* KSg = a.ks + (long long)bh * a.nkp * NB;
    const uint8_t* Vg = a.v8t + (long long)bh * a.ntile * D * 64;
    const uint8_t* VSg = a.vs + (long long)bh * a.ntile * D * 2;
    const unsigned lds_k = (unsigned)(size_t)(lds_char*)smem, lds_v = lds_k + NST * KTB;
    const unsigned lds_ks = (unsigned)(size_t)(lds_char*)&sks[0][0];
    const unsigned lds_vs = (unsigned)(size_t)(lds_char*)&svs[0][0];
    // this wave's share of a tile: K8 rows 32*grp + 8*wg + lane/8 (chunk lane%8),
    // V8T rows 64*grp + 16*wg + lane/4 (chunk lane%4); wave 0 of group 0 the
    // key scales, wave 0 of group 1 the value scales
    const int krow_l = 32 * grp + 8 * wg + (lane >> 3), vrow_l = 64 * grp + 16 * wg + (lane >> 2);
    const unsigned kvo = (unsigned)krow_l * D + (unsigned)(((lane & 7) ^ k8_swz(krow_l)) * 16);
    const unsigned vvo = (unsigned)vrow_l * 64 + (unsigned)(((lane & 3) ^ v8_swz(vrow_l)) * 16);
    auto issue_k = [&](int stage, int tile) {
      dma16(__builtin_amdgcn_readfirstlane(lds_k + stage * KTB + (32 * grp + 8 * wg) * D), Kg,
            (unsigned)tile * KTB + kvo);
      if (wg == 0 && grp == 0) dma4(lds_ks + stage * BN * 4, KSg, (unsigned)tile * BN * NB + (unsigned)lane * 4u);
    };
    auto issue_v = [&](int stage, int tile) {
      dma16(__builtin_amdgcn_readfirstlane(lds_v + stage * VTB + (64 * grp + 16 * wg) * 64), Vg,
            (unsigned)tile * VTB + vvo);
      if (wg == 0 && grp == 1) dma4(lds_vs + stage * D * 2, VSg, (unsigned)tile * D * 2 + (unsigned)lane * 4u);
    };

    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.f;   // m_ref: exp2 domain, a whole number once set
    const float sc = a.scale_log2;

    struct STile { f32x16 t[2]; };
    // X: 4 P.V MFMAs, then 4 K.Q^T MFMAs; P.V operands read first, each K.Q^T
    // operand pair read one MFMA ahead
    auto pv_qk = [&](int vstage, const v8i& pB, int kstage) -> STile {
      const char* V0 = smem + NST * KTB + vstage * VTB;
      const char* K0 = smem + kstage * KTB;
      v8i va[NT], ka[4];
      int vsc[NT], ksc[4];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = 32 * t + l32;
        const char* vp = V0 + d * 64;
        va[t] = lds_operand(vp + (((2 * h) ^ v8_swz(d)) * 16), vp + (((2 * h + 1) ^ v8_swz(d)) * 16));
        vsc[t] = (int)((svs[vstage][d >> 1] >> (16 * (d & 1) + 8 * h)) & 0xffu);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int krow = half * 32 + l32;
        const char* kp = K0 + krow * D;
        const uint32_t ksw = sks[kstage][krow];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          ka[2 * half + u] = lds_operand(kp + (((4 * u + h) ^ k8_swz(krow)) * 16), kp + (((4 * u + 2 + h) ^ k8_swz(krow)) * 16));
          ksc[2 * half + u] = (int)((ksw >> (8 * (2 * u + h))) & 0xffu);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[t], pB, acc[t], 0, 0, 0, vsc[t], 0, 127);
      STile S;
      S.t[0] = f32x16{};
      S.t[1] = f32x16{};
#pragma unroll
      for (int m = 0; m < 4; ++m)
        S.t[m >> 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[m], qB[m & 1], S.t[m >> 1], 0, 0, 0, ksc[m], 0,
                                                                     qS[m & 1]);
      constexpr int kMFMA = 0x8, kDSR = 0x100;
      __builtin_amdgcn_sched_group_barrier(kDSR, 2 * NT + 2, 0);
#pragma unroll
      for (int m = 0; m < 7; ++m) {
        __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
        if (m < 3) __builtin_amdgcn_sched_group_barrier(kDSR, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
      return S;
    };

    // softmax of tile j (exp2 domain, integer reference max): probabilities
    // first against the current reference, the row max and the move rule only
    // when a lane's tile sum leaves [0, 2^7] (a probability above 2^8, where
    // isa_flash_fp8_kernel moves the reference, implies that)
    auto softmax = [&](int j, STile St, v8i& pB) {
      const int t0 = (t_begin + j) * BN;
      float x[32];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[16 * half + r] = St.t[half][r];
      if (t0 + BN > n_valid) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int key = 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * h + (i & 3);
          if (t0 + key >= n_valid) x[i] = -INFINITY;
        }
      }
      auto probs = [&]() -> float {
        float psum = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(x[4 * g + e], sc, -m_ref));
            psum += p[e];
          }
          pB[g] = (int)pack4_fp8(p[0], p[1], p[2], p[3]);
        }
        return psum;
      };
      float psum = probs();
      if (__ballot(!(psum <= 128.f))) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 32; ++i) mx = fmaxf(mx, x[i]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sc;
        const bool move = mx > m_ref + 8.0f;
        if (__ballot(move)) {
          const float m_new = move ? ceilf(mx) : m_ref;
          const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] *= alpha;
          m_ref = m_new;
          psum = probs();
        }
      }
      l_run += psum;
    };
    auto phase_barrier = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    const int t_last = t_begin + nt - 1;
    auto tl = [&](int j) { return min(t_begin + j, t_last); };
    if (nt > 0) {
      issue_k(0, tl(0));
      issue_k(1, tl(1));
      issue_k(2, tl(2));
      issue_v(0, tl(0));
      issue_v(1, tl(1));
      // V stage 3 is first loaded in step 1; step 0 multiplies it (as zeros) by P = 0
      u32x4* vz = (u32x4*)(smem + NST * KTB + 3 * VTB);
      for (int q = tid; q < VTB / 16; q += 512) vz[q] = u32x4{0u, 0u, 0u, 0u};
      if (tid < D / 2) svs[3][tid] = 0u;
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
      phase_barrier();
      if (grp == 1) phase_barrier();   // group 1 runs one phase behind group 0
      STile S = {};
      v8i pB = {};
      auto step = [&](int j) {
        const int Z = j & 3;
        // X_j (step nt computes an S that is never used)
        __builtin_amdgcn_s_setprio(3);
        S = pv_qk((Z + 3) & 3, pB, Z);
        __builtin_amdgcn_sched_barrier(0);
        // loads past the last tile re-read it into the stage the schedule
        // frees for tile j+3 / j+2 and are never read
        issue_k((Z + 3) & 3, tl(j + 3));
        issue_v((Z + 2) & 3, tl(j + 2));
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        phase_barrier();
        // Y_j
        if (j < nt) softmax(j, S, pB);
        // the loads of X_{j-1} have landed before the barrier that closes Y_j
        // (wave 0 of each group also loads one scale slice per step)
        if (wg == 0) __builtin_amdgcn_s_waitcnt(0x0f73);   // vmcnt(3)
        else __builtin_amdgcn_s_waitcnt(0x0f72);           // vmcnt(2)
        phase_barrier();
      };
      for (int j = 0; j <= nt; ++j) step(j);
      __builtin_amdgcn_s_waitcnt(0x0f70);   // no load into this workgroup's LDS outlives it
      if (grp == 0) phase_barrier();   // balances group 1's extra barrier
    }

    // ---- epilogue (as isa_flash_fp8_kernel's)
    const float l_tot = l_run + wave_shfl_xor(l_run, 32);
    if (part < 0) {
      if (qrow < 0) continue;
      const float inv = 1.0f / l_tot;
      bf16_t* op = (bf16_t*)a.O + rm_head(a.rmo, bh) + (long long)qrow * a.rmo.sn;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2*)(op + 32 * t + 8 * g + 4 * h) =
              u32x2{pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv),
                    pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv)};
      if (a.lse && h == 0) a.lse[(long long)bh * a.Ns + qrow] = m_ref + __builtin_log2f(l_tot);
    } else {
      // part `part` of range-phase row tile Rs: [Rs][sk_P][BM][D]
      const long long prow = ((long long)Rs * a.sk_P + part) * BM + w * 32 + l32;
      bf16_t* po = a.part_o + prow * D;
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2*)(po + 32 * t + 8 * g + 4 * h) =
              u32x2{pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv),
                    pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv)};
      if (h == 0) *(float2*)(a.part_ml + prow * 2) = float2{m_ref / sc, l_tot};
    }
  }  // items
}

// ---------------------------------------------------------------------------

static Fp8Args fp8_args(const Layout& L, const Fp8Layout& F, const Bufs& B, char* fws) {
  Fp8Args a = {};
  a.Q = B.Q; a.O = B.O; a.K = B.K; a.V = B.V;
  a.rmq = L.q; a.rmo = L.o; a.rmk = L.k; a.rmv = L.v;
  a.ctx_rows = (const int*)(B.ws + L.off_ctxrows);
  a.kept = (const int*)(B.ws + L.off_kept);
  a.ctx_tok = L.ctx_tok;
  a.kc = L.kc; a.nb_c = L.nb_c; a.b = L.b; a.tail_c = L.tail_c;
  a.k8 = (uint8_t*)(fws + F.off_k8);
  a.ks = (uint8_t*)(fws + F.off_ks);
  a.v8t = (uint8_t*)(fws + F.off_v8t);
  a.vs = (uint8_t*)(fws + F.off_vs);
  a.nkp = F.nkp; a.ntile = F.ntile;
  a.q_list = (const int*)(B.ws + L.off_fullq);
  a.q_k = L.kq; a.nb_s = L.nb_s;
  a.lse = (float*)(B.ws + L.off_lse);
  a.part_o = (bf16_t*)(B.ws + L.off_part_o);
  a.part_ml = (float*)(B.ws + L.off_part_ml);
  a.nsplit = L.full_splits;
  a.Ns = L.Ns; a.Nk = L.Nk;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)L.d));
  return a;
}

template <int D>
static hipError_t fp8_t(const Layout& L, const Fp8Layout& F, const Bufs& B, char* fws, bool pack, hipStream_t s) {
  Fp8Args a = fp8_args(L, F, B, fws);
  if (pack) {
    hipLaunchKernelGGL((isa_fp8_pack_kernel<D>), dim3((unsigned)F.ntile, (unsigned)L.BH), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  a.row_tiles = (int)((L.full_rows + kFlashRows - 1) / kFlashRows);
  const int ntiles = (int)((L.Ns + L.ctx_tok + 63) / 64);
  a.tiles_per_split = (ntiles + a.nsplit - 1) / a.nsplit;
  const long long nwg = (long long)a.row_tiles * L.BH * a.nsplit;
  if (nwg == 0) return hipSuccess;
  a.n_wg = (int)nwg;
  if constexpr (D == 128 && kFlashWaves == 8) {
    // the stream-K split of the bf16 route (the layout's): whole row tiles in
    // a.sk_K rounds of grid workgroups, then a.sk_G ranges
    const long long R = (long long)a.row_tiles * L.BH, grid = L.sk_grid;
    a.sk_K = L.sk_rounds;
    a.sk_G = L.sk_G;
    a.sk_P = L.sk_P;
    a.sk_R0 = (int)(grid * a.sk_K);
    a.sk_grid = (int)grid;
    a.sk_q = (int)(R / 8);
    a.sk_x = (int)(R % 8);
    a.sk_T = ntiles;
    a.sk_U = (R - a.sk_R0) * ntiles;
    if (grid <= 0 || grid % 8 != 0 || a.sk_K < 0 || a.sk_R0 > R || (a.sk_U > 0) != (a.sk_G > 0) || a.sk_U < a.sk_G ||
        a.sk_P < 1 || a.sk_P > kMaxSplits)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(isa_flash_fp8_pp_kernel, dim3((unsigned)(a.sk_K > 0 ? grid : a.sk_G)), dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL((isa_flash_fp8_kernel<D>), dim3((unsigned)nwg), dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fp8(const Layout& L, const Fp8Layout& F, const Bufs& B, char* fws, bool pack, hipStream_t s) {
  return L.d == 128 ? fp8_t<128>(L, F, B, fws, pack, s) : fp8_t<64>(L, F, B, fws, pack, s);
}

}  // namespace isa
