// Context saliency (pre-selection score) on MFMA.
//
// Per the abstract of "Lightning Unified Video Editing via In-Context Sparse
// Attention", the context tokens matter far less to the source queries than
// the source tokens do, so the least salient context blocks are dropped
// before attention.  Saliency of
// context block c is read here as the probability mass that the pooled
// source queries put on it under the n-weighted softmax over every pooled
// key block:
//     P_ij  = n_j exp(qbar_i . kbar_j / sqrt d) / sum_j' n_j' exp(...)
//     sal_c = sum_i P_{i, nb_s + c}.
//
// One workgroup (8 waves) per 32 pooled queries of one head.  Logits
// L^T = Kbar Qbar^T come from 32x32x16 bf16 MFMAs on a two-part split of the
// fp32 pooled vectors (hi = bf16(x), lo = bf16(x - hi); hi*hi + hi*lo +
// lo*hi, about 2^-17 relative per product).  Pass 1: each lane keeps the
// running max and the n-weighted sum of exp for its query over its keys (sum
// in fp64); lanes and waves are combined in a fixed order.  Pass 2 recomputes
// the context logits, forms the probabilities (exp of a centred fp32
// argument, fp64 products and sums) and sums them over the 32 queries through
// LDS in query order.  Each workgroup writes the column sums of its queries;
// the select kernel adds the workgroups in order, so the result is
// deterministic.
#include "isa_device.h"
#include "isa_kernels.h"

namespace isa {

constexpr int kSalCtxCache = 512;   // context blocks whose logits pass 2 takes from LDS

struct SalArgs {
  const float* qbar;
  const float* kbar;
  double* salp;
  int nb_s, nb_c, M, b, tail_s, tail_c, sal_tiles;
  float inv_sqrt_d;
};

__device__ __forceinline__ double block_count(int j, int nb_s, int nb_c, int b, int tail_s, int tail_c) {
  if (j < nb_s) return j == nb_s - 1 ? tail_s : b;
  return (j - nb_s) == nb_c - 1 ? tail_c : b;
}

// 8 fp32 values -> bf16 hi and lo operands
__device__ __forceinline__ void split8(const float* src, bf16x8& hi, bf16x8& lo) {
  const f32x4 a = *(const f32x4*)src;
  const f32x4 b = *(const f32x4*)(src + 4);
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)v[j];
    hi[j] = h;
    lo[j] = (__bf16)(v[j] - (float)h);
  }
}

template <int D>
__global__ __launch_bounds__(512) void isa_saliency_kernel(SalArgs a) {
  constexpr int R = kSalRows;  // 32 pooled queries
  constexpr int NW = 8;
  __shared__ double red_m[NW][R], red_s[NW][R];
  __shared__ double pt[NW][32][R + 1];  // per wave: [key][query] probabilities
  // context logits of pass 1, [context block][query], reused by pass 2 when
  // they fit (nb_c <= kSalCtxCache); otherwise pass 2 recomputes them
  __shared__ float lctx[kSalCtxCache][R];
  const bool cache = a.nb_c <= kSalCtxCache;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int tile = blockIdx.x;
  const long long bh = blockIdx.y;
  const int i0 = tile * R;
  const int nr = min(R, a.nb_s - i0);
  const float* kb = a.kbar + bh * (long long)a.M * D;

  // B operands: pooled query l32 (zero when past the end), d = 16 s + 8 h + j
  bf16x8 qh[D / 16], ql[D / 16];
  {
    const int q = l32 < nr ? i0 + l32 : i0;
    const float* qp = a.qbar + (bh * a.nb_s + q) * (long long)D + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      split8(qp + 16 * s, qh[s], ql[s]);
      if (l32 >= nr) { qh[s] = bf16x8{}; ql[s] = bf16x8{}; }
    }
  }
  // logits of 32 keys starting at key k0: lane (l32, h) gets keys
  // k0 + 8*(r/4) + 4*h + r%4 of its query, r = 0..15 (keys past M are garbage)
  auto logits = [&](int k0) -> f32x16 {
    const int key = min(k0 + l32, a.M - 1);
    const float* kp = kb + (long long)key * D + 8 * h;
    // two accumulators (even and odd d steps) halve the MFMA dependency chain
    f32x16 S0 = f32x16{}, S1 = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      bf16x8 kh, kl;
      split8(kp + 16 * s, kh, kl);
      f32x16& S = (s & 1) ? S1 : S0;
      S = mma32(kh, qh[s], S);
      S = mma32(kh, ql[s], S);
      S = mma32(kl, qh[s], S);
    }
    return (S0 + S1) * a.inv_sqrt_d;
  };
  auto key_of = [&](int k0, int r) { return k0 + 8 * (r >> 2) + 4 * h + (r & 3); };

  // ---- pass 1: per-query max and n-weighted sum over every key block
  float m = -INFINITY;
  double s = 0.0;
  for (int k0 = 32 * w; k0 < a.M; k0 += 32 * NW) {
    const f32x16 L = logits(k0);
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key_of(k0, r) < a.M) tmax = fmaxf(tmax, L[r]);
    if (cache && k0 + 32 > a.nb_s) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = key_of(k0, r);
        if (j >= a.nb_s && j < a.M) lctx[j - a.nb_s][l32] = L[r];
      }
    }
    if (tmax > m) {
      if (m != -INFINITY) s *= (double)__builtin_amdgcn_exp2f((m - tmax) * 1.4426950408889634f);
      m = tmax;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = key_of(k0, r);
      if (j < a.M)
        s += block_count(j, a.nb_s, a.nb_c, a.b, a.tail_s, a.tail_c) *
             (double)__builtin_amdgcn_exp2f((L[r] - m) * 1.4426950408889634f);
    }
  }
  // combine the two lane halves, then the waves, in a fixed order
  auto combine = [](float& m1, double& s1, float m2, double s2) {
    const float mm = fmaxf(m1, m2);
    double t = 0.0;
    if (m1 != -INFINITY) t += s1 * (double)__builtin_amdgcn_exp2f((m1 - mm) * 1.4426950408889634f);
    if (m2 != -INFINITY) t += s2 * (double)__builtin_amdgcn_exp2f((m2 - mm) * 1.4426950408889634f);
    m1 = mm;
    s1 = t;
  };
  {
    const float m2 = __shfl_xor(m, 32, 64);
    const double s2 = __shfl_xor(s, 32, 64);
    if (h == 0) combine(m, s, m2, s2);
    else { float mm = m2; double ss = s2; combine(mm, ss, m, s); m = mm; s = ss; }
  }
  if (h == 0) {
    red_m[w][l32] = m;
    red_s[w][l32] = s;
  }
  __syncthreads();
  float mq = (float)red_m[0][l32];
  double sq = red_s[0][l32];
#pragma unroll
  for (int v = 1; v < NW; ++v) combine(mq, sq, (float)red_m[v][l32], red_s[v][l32]);
  const double inv_s = 1.0 / sq;

  // ---- pass 2: probabilities on the context blocks, summed over the queries
  double* out = a.salp + (bh * a.sal_tiles + tile) * (long long)a.nb_c;
  const int nct = (a.nb_c + 31) / 32;
  for (int ct0 = 0; ct0 < nct; ct0 += NW) {
    const int ct = ct0 + w;
    if (ct < nct) {
      const int k0 = a.nb_s + 32 * ct;
      f32x16 L;
      if (cache) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = key_of(k0, r);
          L[r] = j < a.M ? lctx[j - a.nb_s][l32] : 0.f;
        }
      } else {
        L = logits(k0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = key_of(k0, r);
        double p = 0.0;
        if (j < a.M && l32 < nr)
          p = block_count(j, a.nb_s, a.nb_c, a.b, a.tail_s, a.tail_c) *
              (double)__builtin_amdgcn_exp2f((L[r] - mq) * 1.4426950408889634f) * inv_s;
        pt[w][8 * (r >> 2) + 4 * h + (r & 3)][l32] = p;
      }
    }
    __syncthreads();
    // one thread per (wave tile, key): add the 32 queries in order
    if (tid < 32 * NW) {
      const int v = tid >> 5, kk = tid & 31;
      const int c = 32 * (ct0 + v) + kk;
      if (ct0 + v < nct && c < a.nb_c) {
        double col = 0.0;
        for (int q = 0; q < R; ++q) col += pt[v][kk][q];
        out[c] = col;
      }
    }
    __syncthreads();
  }
}

template <int D>
static hipError_t launch_sal_t(const Layout& L, const Bufs& B, hipStream_t s) {
  SalArgs a;
  a.qbar = (const float*)(B.ws + L.off_qbar);
  a.kbar = (const float*)(B.ws + L.off_kbar);
  a.salp = (double*)(B.ws + L.off_salp);
  a.nb_s = L.nb_s; a.nb_c = L.nb_c; a.M = L.M; a.b = L.b;
  a.tail_s = L.tail_s; a.tail_c = L.tail_c; a.sal_tiles = L.sal_tiles;
  a.inv_sqrt_d = 1.0f / sqrtf((float)D);
  hipLaunchKernelGGL((isa_saliency_kernel<D>), dim3(L.sal_tiles, (unsigned)L.BH), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_saliency(const Layout& L, const Bufs& B, hipStream_t s) {
  if (L.nb_c == 0) return hipSuccess;
  return L.d == 128 ? launch_sal_t<128>(L, B, s) : launch_sal_t<64>(L, B, s);
}

}  // namespace isa
