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
//
// Two launches: the pooling pass (source Q, every K block, source V) before
// the saliency, and, after the context selection, the packing pass, which
// pools V of the kept context blocks and writes the packed kept key set of
// the pooled attention in the same wave.
#include "isa_device.h"
#include "isa_kernels.h"

namespace isa {

struct PoolArgs {
  const void* Q;
  const void* K;
  const void* V;
  RowMap rmq, rmk, rmv;  // element strides of Q, K, V
  float* qbar;
  float* kbar;
  float* vbar;
  const int* kept;  // packing pass: [BH][kc]
  void* pkhi;       // packing pass: [BH][mk_pad][D] in the input type
  bf16_t* pklo;     // (bf16 inputs only)
  void* pv;
  float* pbias;     // [BH][mk_pad]
  int Ns, Nc, Nk, b, nb_s, nb_c, M, kc, mk, mk_pad, tail_s, tail_c;
  int tasks_per_head;
  long long total_tasks;
};

// Mean of `rows` rows of d elements from `base`, rows `rs` bytes apart
// (16-byte chunk column c = lane % CPR of each row): every lane of column c
// ends with the sums.  NT: non-temporal loads (the streaming pass reads
// every input row once; the hint keeps its 0.4 GB from cycling through the
// caches).
template <typename T, int D, bool NT>
__device__ __forceinline__ void pool_rows(const char* base, int rows, unsigned rs, float* acc) {
  constexpr int ES = sizeof(T);
  constexpr int CPR = D * ES / 16;     // 16-byte chunks per row
  constexpr int RG = 64 / CPR;         // rows in flight per wave
  constexpr int EPC = 16 / ES;         // elements per chunk
  const int lane = threadIdx.x & 63;
  const int c = lane % CPR, rg = lane / CPR;
  // Row offsets: rows < 2^24 and rs < 2^24, and a head spans less than 2^31
  // bytes.  The streaming pass (NT) loads with non-temporal global loads,
  // a row past the block not at all; the packing pass loads through a
  // buffer descriptor of the block's rows (anything past it reads as zero),
  // unconditionally.  (Measured on the video-DiT layer: each form is the
  // faster one for its pass.)
  const unsigned coff = (unsigned)c * 16u;
  // (every value of the descriptor is wave-uniform: readfirstlane says so;
  // the streaming pass does not use it)
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform64((long long)base), (short)0,
      (int)__builtin_amdgcn_readfirstlane((unsigned)(rows - 1) * rs + D * ES), 0x00020000);
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  // BATCH rows per lane are loaded before any is added (bytes in flight);
  // each lane adds its rows in increasing order, a row past the block as
  // zero.
  constexpr int BATCH = 16;
  for (int r0b = rg; r0b < rows; r0b += RG * BATCH) {
    u32x4 v[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int r = r0b + i * RG;
      if constexpr (NT) {
        const u32x4* src = (const u32x4*)(base + (long long)r * rs + coff);
        v[i] = r < rows ? __builtin_nontemporal_load(src) : u32x4{0u, 0u, 0u, 0u};
      } else {
        const unsigned off = __umul24((unsigned)r, rs) + coff;
        const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
        v[i] = r < rows ? x : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
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
}

// First row and row count of pooled block blk (source blocks, then context).
__device__ __forceinline__ void block_rows(const PoolArgs& a, int blk, int* r0, int* rows) {
  if (blk < a.nb_s) {
    *r0 = blk * a.b;
    *rows = min(a.b, a.Ns - *r0);
  } else {
    const int c = blk - a.nb_s;
    *r0 = a.Ns + c * a.b;
    *rows = min(a.b, a.Nc - c * a.b);
  }
}

// Pooling pass: task t of a head is source query block t (t < nb_s), key
// block t - nb_s (every one of the M blocks) or source value block
// t - nb_s - M.
template <typename T, int D>
__global__ __launch_bounds__(256) void isa_pool_kernel(PoolArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int CPR = D * ES / 16;
  constexpr int EPC = 16 / ES;
  const int lane = threadIdx.x & 63;
  // (the wave index through readfirstlane: the task is wave-uniform, so its
  // row addresses are a scalar base plus per-lane offsets)
  const long long task = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (task >= a.total_tasks) return;
  const long long bh = task / a.tasks_per_head;
  const int t = (int)(task - bh * a.tasks_per_head);
  // (the row map is selected by value: a pointer into the argument block
  // would make the compiler copy the whole block to scratch memory)
  const void* src;
  RowMap m;
  float* dst;
  int blk;
  if (t < a.nb_s) {
    src = a.Q; m = a.rmq; dst = a.qbar + (bh * a.nb_s + t) * D; blk = t;
  } else if (t < a.nb_s + a.M) {
    blk = t - a.nb_s; src = a.K; m = a.rmk; dst = a.kbar + (bh * a.M + blk) * D;
  } else {
    blk = t - a.nb_s - a.M; src = a.V; m = a.rmv; dst = a.vbar + (bh * a.M + blk) * D;
  }
  int r0, rows;
  block_rows(a, blk, &r0, &rows);
  float acc[EPC];
  pool_rows<T, D, true>((const char*)src + (rm_head(m, bh) + (long long)r0 * m.sn) * ES, rows,
                        (unsigned)m.sn * ES, acc);
  if (lane < CPR) {
    const float n = (float)rows;
#pragma unroll
    for (int e = 0; e < EPC; ++e) dst[lane * EPC + e] = acc[e] / n;
  }
}

// Packing pass: task p of a head is row p of the packed kept key set of the
// pooled (Taylor / sharpness) attention -- source block p (p < nb_s), kept
// context block kept[p - nb_s] (p < mk), or padding (zero, bias -inf).  A
// kept context block's V rows are pooled here (its K was pooled in the
// first pass); source blocks take both from the first pass.  The bias is
// log2 n_j, the count weight of the n-weighted softmax in the exp2 domain.
// bf16 inputs store each pooled key as hi = bf16(k) and lo = bf16(k - hi):
// the two bf16 products with a bf16 query carry the logit to about 2^-17
// relative, well inside what the sharpness selection needs.
template <typename T, int D>
__global__ __launch_bounds__(256) void isa_pool_pack_kernel(PoolArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int CPR = D * ES / 16;
  constexpr int EPC = 16 / ES;
  const int lane = threadIdx.x & 63;
  const long long task = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (task >= a.total_tasks) return;
  const long long bh = task / a.mk_pad;
  const int p = (int)(task - bh * a.mk_pad);
  int j = -1;   // pooled block of the row
  if (p < a.nb_s) {
    j = p;
  } else if (p < a.mk) {
    const int c = a.kept[bh * a.kc + (p - a.nb_s)];
    j = (c >= 0 && c < a.nb_c) ? a.nb_s + c : -1;   // (always, for a well-formed list)
  }
  float v[EPC], k[EPC];
  int rows = 0;
  if (j >= 0) {
    int r0;
    block_rows(a, j, &r0, &rows);
    const float* vb = a.vbar + (bh * a.M + j) * D;
    if (j >= a.nb_s) {
      float acc[EPC];
      pool_rows<T, D, false>((const char*)a.V + (rm_head(a.rmv, bh) + (long long)r0 * a.rmv.sn) * ES, rows,
                             (unsigned)a.rmv.sn * ES, acc);
      const float n = (float)rows;
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[e] = acc[e] / n;
      if (lane < CPR) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) ((float*)vb)[lane * EPC + e] = v[e];
      }
    } else if (lane < CPR) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[e] = vb[lane * EPC + e];
    }
    if (lane < CPR) {
      const float* kb = a.kbar + (bh * a.M + j) * D;
#pragma unroll
      for (int e = 0; e < EPC; ++e) k[e] = kb[lane * EPC + e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPC; ++e) v[e] = k[e] = 0.f;
  }
  if (lane < CPR) {
    const long long dst = (bh * a.mk_pad + p) * D + lane * EPC;
    if constexpr (ES == 2) {
      u32x4 hi, lo, vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16_t h0 = to_bf16(k[2 * e]), h1 = to_bf16(k[2 * e + 1]);
        hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[e] = pack_bf16x2(k[2 * e] - to_f32(h0), k[2 * e + 1] - to_f32(h1));
        vv[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
      }
      *(u32x4*)((bf16_t*)a.pkhi + dst) = hi;
      *(u32x4*)(a.pklo + dst) = lo;
      *(u32x4*)((bf16_t*)a.pv + dst) = vv;
    } else {
      *(f32x4*)((float*)a.pkhi + dst) = f32x4{k[0], k[1], k[2], k[3]};
      *(f32x4*)((float*)a.pv + dst) = f32x4{v[0], v[1], v[2], v[3]};
    }
  }
  if (lane == 0) {
    float bias = -INFINITY;
    if (j >= 0) {
      const int n = j < a.nb_s ? (j == a.nb_s - 1 ? a.tail_s : a.b) : ((j - a.nb_s) == a.nb_c - 1 ? a.tail_c : a.b);
      bias = log2f((float)n);
    }
    a.pbias[bh * a.mk_pad + p] = bias;
  }
}

static PoolArgs pool_args(const Layout& L, const Bufs& B) {
  PoolArgs a;
  a.Q = B.Q; a.K = B.K; a.V = B.V;
  a.rmq = L.q; a.rmk = L.k; a.rmv = L.v;
  a.qbar = (float*)(B.ws + L.off_qbar);
  a.kbar = (float*)(B.ws + L.off_kbar);
  a.vbar = (float*)(B.ws + L.off_vbar);
  a.kept = (const int*)(B.ws + L.off_kept);
  a.pkhi = B.ws + L.off_pkhi;
  a.pklo = (bf16_t*)(B.ws + L.off_pklo);
  a.pv = B.ws + L.off_pv;
  a.pbias = (float*)(B.ws + L.off_pbias);
  a.Ns = L.Ns; a.Nc = L.Nc; a.Nk = L.Nk; a.b = L.b;
  a.nb_s = L.nb_s; a.nb_c = L.nb_c; a.M = L.M; a.kc = L.kc; a.mk = L.mk; a.mk_pad = L.mk_pad;
  a.tail_s = L.tail_s; a.tail_c = L.tail_c;
  return a;
}

template <typename T, int D>
static hipError_t launch_pool_t(const Layout& L, const Bufs& B, bool pack, hipStream_t s) {
  PoolArgs a = pool_args(L, B);
  a.tasks_per_head = pack ? L.mk_pad : 2 * L.nb_s + L.M;
  a.total_tasks = (long long)a.tasks_per_head * L.BH;
  if (a.total_tasks == 0) return hipSuccess;
  const long long grid = (a.total_tasks + 3) / 4;
  if (pack) hipLaunchKernelGGL((isa_pool_pack_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((isa_pool_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

static hipError_t launch_pool_any(const Layout& L, const Bufs& B, bool pack, hipStream_t s) {
  if (L.es == 2) return L.d == 128 ? launch_pool_t<bf16_t, 128>(L, B, pack, s) : launch_pool_t<bf16_t, 64>(L, B, pack, s);
  return L.d == 128 ? launch_pool_t<float, 128>(L, B, pack, s) : launch_pool_t<float, 64>(L, B, pack, s);
}

hipError_t launch_pool(const Layout& L, const Bufs& B, hipStream_t s) { return launch_pool_any(L, B, false, s); }

hipError_t launch_pool_pack(const Layout& L, const Bufs& B, hipStream_t s) { return launch_pool_any(L, B, true, s); }

}  // namespace isa
