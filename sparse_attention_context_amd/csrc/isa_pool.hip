// Block mean-pool of Q, K and V (HBM-streaming).
//
// Pooled blocks are the basis of the method's cheap paths: the 0-th order
// Taylor attention replaces every key of a block by the block mean (Lightning
// Unified Video Editing via In-Context Sparse Attention, English abstract),
// and saliency and sharpness are read off the same pooled softmax.
//
// One wave per block.  A row of d elements is CPR 16-byte chunks; the 64
// lanes cover 64/CPR rows at a time, each lane summing one chunk column in
// fp32, then a fixed xor-shuffle tree adds the row groups (deterministic).
#include "isa_device.h"
#include "isa_kernels.h"

namespace isa {

struct PoolArgs {
  const void* Q;
  const void* K;
  const void* V;
  float* qbar;
  float* kbar;
  float* vbar;
  const int* kept;  // pass 1
  int Ns, Nc, Nk, b, nb_s, nb_c, M, kc;
  int tasks_per_head;
  int pass;
  long long total_tasks;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void isa_pool_kernel(PoolArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int CPR = D * ES / 16;     // 16-byte chunks per row
  constexpr int RG = 64 / CPR;         // rows in flight per wave
  constexpr int EPC = 16 / ES;         // elements per chunk
  const int lane = threadIdx.x & 63;
  const long long task = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= a.total_tasks) return;
  const long long bh = task / a.tasks_per_head;
  int t = (int)(task - bh * a.tasks_per_head);

  // task -> (tensor, block)
  const void* src;
  float* dst;
  int rows, blk;
  long long nrows_head;
  if (a.pass == 0) {
    if (t < a.nb_s) {
      src = a.Q; dst = a.qbar + (bh * a.nb_s + t) * D; blk = t; nrows_head = a.Ns;
    } else if (t < a.nb_s + a.M) {
      blk = t - a.nb_s; src = a.K; dst = a.kbar + (bh * a.M + blk) * D; nrows_head = a.Nk;
    } else {
      blk = t - a.nb_s - a.M; src = a.V; dst = a.vbar + (bh * a.M + blk) * D; nrows_head = a.Nk;
    }
  } else {
    const int kc_blk = a.kept[bh * a.kc + t];
    if (kc_blk < 0 || kc_blk >= a.nb_c) return;  // never for a well-formed list
    blk = a.nb_s + kc_blk;
    src = a.V; dst = a.vbar + (bh * a.M + blk) * D; nrows_head = a.Nk;
  }
  int r0;
  if (blk < a.nb_s) {
    r0 = blk * a.b;
    rows = min(a.b, a.Ns - r0);
  } else {
    const int c = blk - a.nb_s;
    r0 = a.Ns + c * a.b;
    rows = min(a.b, a.Nc - c * a.b);
  }

  const int c = lane % CPR, rg = lane / CPR;
  const char* base = (const char*)src + ((bh * nrows_head + r0) * D) * ES + c * 16;
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  // BATCH rows per lane are loaded before any is added (bytes in flight);
  // each lane still adds its rows in increasing order
  constexpr int BATCH = 16;
  for (int r0b = rg; r0b < rows; r0b += RG * BATCH) {
    u32x4 v[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int r = r0b + i * RG;
      v[i] = r < rows ? *(const u32x4*)(base + (long long)r * D * ES) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      if (r0b + i * RG >= rows) break;
      if constexpr (ES == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(v[i][e] << 16);
          acc[2 * e + 1] += __uint_as_float(v[i][e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[i][e]);
      }
    }
  }
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += wave_shfl_xor(acc[e], off);
  if (rg == 0) {
    const float n = (float)rows;
#pragma unroll
    for (int e = 0; e < EPC; ++e) dst[c * EPC + e] = acc[e] / n;
  }
}

template <typename T, int D>
static hipError_t launch_pool_t(const Layout& L, const Bufs& B, int pass, hipStream_t s) {
  PoolArgs a;
  a.Q = B.Q; a.K = B.K; a.V = B.V;
  a.qbar = (float*)(B.ws + L.off_qbar);
  a.kbar = (float*)(B.ws + L.off_kbar);
  a.vbar = (float*)(B.ws + L.off_vbar);
  a.kept = (const int*)(B.ws + L.off_kept);
  a.Ns = L.Ns; a.Nc = L.Nc; a.Nk = L.Nk; a.b = L.b;
  a.nb_s = L.nb_s; a.nb_c = L.nb_c; a.M = L.M; a.kc = L.kc;
  a.pass = pass;
  a.tasks_per_head = pass == 0 ? (2 * L.nb_s + L.M) : L.kc;
  a.total_tasks = (long long)a.tasks_per_head * L.BH;
  if (a.total_tasks == 0) return hipSuccess;
  const long long grid = (a.total_tasks + 3) / 4;
  hipLaunchKernelGGL((isa_pool_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pool(const Layout& L, const Bufs& B, int pass, hipStream_t s) {
  if (L.es == 2) return L.d == 128 ? launch_pool_t<bf16_t, 128>(L, B, pass, s) : launch_pool_t<bf16_t, 64>(L, B, pass, s);
  return L.d == 128 ? launch_pool_t<float, 128>(L, B, pass, s) : launch_pool_t<float, 64>(L, B, pass, s);
}

}  // namespace isa
