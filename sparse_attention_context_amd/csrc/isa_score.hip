// Context saliency (pre-selection score).
//
// The abstract of "Lightning Unified Video Editing via In-Context Sparse
// Attention" observes that context tokens carry much lower saliency than
// source tokens and prunes redundant context before attention.  Saliency of
// context block c is read here as the probability mass that the pooled
// source queries put on it under the n-weighted softmax over every pooled
// key block:
//     P_ij  = n_j exp(qbar_i . kbar_j / sqrt d) / sum_j' n_j' exp(...)
//     sal_c = sum_i P_{i, nb_s + c}.
//
// One workgroup per 16 pooled queries of one head.  Logits are fp32 dot
// products in a fixed order; the normaliser, the probabilities and the
// column sums are fp64 (the scores decide a discrete selection, so they are
// kept far more accurate than the 1e-6 the selection is checked to).  Each
// workgroup writes the column sums of its rows; the select kernel adds the
// partials in workgroup order, so the result is deterministic.
#include "isa_device.h"
#include "isa_kernels.h"

namespace isa {

struct SalArgs {
  const float* qbar;
  const float* kbar;
  double* salp;
  int nb_s, nb_c, M, b, tail_s, tail_c, sal_tiles;
  float inv_sqrt_d;
};

template <int D>
__device__ __forceinline__ void pooled_logits(const float* __restrict__ krow, const float (*qs)[D],
                                              float* l, float inv_sqrt_d) {
  constexpr int R = kSalRows;
#pragma unroll
  for (int r = 0; r < R; ++r) l[r] = 0.f;
  for (int c0 = 0; c0 < D; c0 += 16) {
    float kv[16];
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 v = *(const float4*)(krow + c0 + e);
      kv[e] = v.x; kv[e + 1] = v.y; kv[e + 2] = v.z; kv[e + 3] = v.w;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 16; ++e) l[r] = fmaf(qs[r][c0 + e], kv[e], l[r]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) l[r] *= inv_sqrt_d;
}

__device__ __forceinline__ double block_count(int j, int nb_s, int nb_c, int b, int tail_s, int tail_c) {
  if (j < nb_s) return j == nb_s - 1 ? tail_s : b;
  return (j - nb_s) == nb_c - 1 ? tail_c : b;
}

template <int D>
__global__ __launch_bounds__(256) void isa_saliency_kernel(SalArgs a) {
  constexpr int R = kSalRows;
  __shared__ float qs[R][D];
  __shared__ double red_m[R][256];
  __shared__ double red_s[R][256];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const long long bh = blockIdx.y;
  const int i0 = tile * R;
  const int nr = min(R, a.nb_s - i0);
  for (int e = tid; e < R * D; e += 256) {
    const int r = e / D, c = e % D;
    qs[r][c] = r < nr ? a.qbar[(bh * a.nb_s + i0 + r) * D + c] : 0.f;
  }
  __syncthreads();
  const float* kb = a.kbar + bh * a.M * D;

  // pass 1: per-row max and n-weighted sum of exp, online, in fp64
  double m[R], s[R];
#pragma unroll
  for (int r = 0; r < R; ++r) { m[r] = -INFINITY; s[r] = 0.0; }
  for (int j = tid; j < a.M; j += 256) {
    float l[R];
    pooled_logits<D>(kb + (long long)j * D, qs, l, a.inv_sqrt_d);
    const double nj = block_count(j, a.nb_s, a.nb_c, a.b, a.tail_s, a.tail_c);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const double lj = l[r];
      if (lj > m[r]) {
        s[r] = s[r] * exp(m[r] - lj) + nj;
        m[r] = lj;
      } else {
        s[r] += nj * exp(lj - m[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) { red_m[r][tid] = m[r]; red_s[r][tid] = s[r]; }
  __syncthreads();
  for (int st = 128; st >= 1; st >>= 1) {
    for (int idx = tid; idx < R * st; idx += 256) {
      const int r = idx / st, i = idx % st;
      const double m1 = red_m[r][i], m2 = red_m[r][i + st];
      const double mm = fmax(m1, m2);
      double sum = 0.0;
      if (mm != -INFINITY) {
        if (m1 != -INFINITY) sum += red_s[r][i] * exp(m1 - mm);
        if (m2 != -INFINITY) sum += red_s[r][i + st] * exp(m2 - mm);
      }
      red_m[r][i] = mm;
      red_s[r][i] = sum;
    }
    __syncthreads();
  }
  double rm[R], rinv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) { rm[r] = red_m[r][0]; rinv[r] = 1.0 / red_s[r][0]; }

  // pass 2: probabilities on context columns, summed over this tile's rows
  double* out = a.salp + (bh * a.sal_tiles + tile) * (long long)a.nb_c;
  for (int c = tid; c < a.nb_c; c += 256) {
    const int j = a.nb_s + c;
    float l[R];
    pooled_logits<D>(kb + (long long)j * D, qs, l, a.inv_sqrt_d);
    const double nj = block_count(j, a.nb_s, a.nb_c, a.b, a.tail_s, a.tail_c);
    double col = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < nr) col += nj * exp((double)l[r] - rm[r]) * rinv[r];
    out[c] = col;
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
  hipLaunchKernelGGL((isa_saliency_kernel<D>), dim3(L.sal_tiles, (unsigned)L.BH), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_saliency(const Layout& L, const Bufs& B, hipStream_t s) {
  if (L.nb_c == 0) return hipSuccess;
  return L.d == 128 ? launch_sal_t<128>(L, B, s) : launch_sal_t<64>(L, B, s);
}

}  // namespace isa
