// Flash-style attention kernels of ISA on gfx950 MFMA, fp32-input path (the
// bf16 path is the pipelined kernel family of isa_flash.hip).
//
// Two routes of "Lightning Unified Video Editing via In-Context Sparse
// Attention" (English abstract) share this kernel:
//  * full attention for the high-error (sharp) query blocks: exact softmax
//    attention over the source tokens and the tokens of the kept context
//    blocks, K/V tiles gathered row by row through the kept-context list;
//  * 0-th order Taylor sparse attention for the other query blocks: the same
//    online softmax over the kept pooled blocks, each carrying the weight n_j
//    (an additive log2 n_j in the exp2 domain).  The peak probability of that
//    pooled softmax -- the query sharpness -- falls out as 1/l, l being the
//    normaliser relative to the running maximum.
// The dense mode (every source query over every key row) is the global
// self-attention of the intelliparadigm.com page, section 1, and is the
// library's own dense baseline.
//
// Layout of the work: a workgroup of 4 waves owns 128 query rows (32 per
// wave) and walks the key tiles of 64 keys.  Per tile each wave computes
// S^T = K Q^T with 32x32 MFMAs (so each lane holds one query and 32 keys),
// does the online softmax in fp32 on exp2, and accumulates O^T = V^T P^T:
// the probabilities in registers already have the layout of the B operand,
// and V is stored transposed in LDS (keys permuted inside each 16-key group
// to match that layout).  K and V^T tiles are double-buffered in LDS with a
// 16-byte XOR swizzle; the next tile's global loads are in flight while the
// current tile is computed.
#include "isa_device.h"
#include "isa_kernels.h"

namespace isa {

enum { KM_DENSE = 0, KM_GATHER = 1, KM_POOLED = 2 };
enum { RM_IDENTITY = 0, RM_TABLE = 1 };

struct AttnArgs {
  const void* Q;
  void* O;
  const void* K;
  const void* V;
  RowMap rmq, rmo, rmk, rmv;  // element strides of Q, O, K, V
  const int* ctx_rows;   // gather: [BH][ctx_tok]
  const int* kept;       // gather: [BH][kc]
  long long ctx_tok;
  int kc, nb_c, b, tail_c;
  const void* pkhi;      // pooled: [BH][mk_pad][D]
  const bf16_t* pklo;
  const void* pv;
  const float* pbias;    // pooled: [BH][mk_pad]
  int mk_pad;
  const int* q_list;     // route block list: [BH][q_k] (table rows)
  int q_k, nb_s;
  long long n_rows;      // virtual rows per head
  float* peak;           // [BH][Ns]
  int Ns, Nk;
  int tiles_per_head;
  int n_wg;
  float scale_log2;      // log2(e) / sqrt(d)
};

template <typename T, int D, int KM, int RM, bool WO, bool WP>
__global__ __launch_bounds__(256) void isa_attn_kernel(AttnArgs a) {
  typedef typename Operand<T>::type Op;
  constexpr int ES = sizeof(T);
  constexpr int BN = 64;
  constexpr int BM = 128;
  constexpr bool POOLED = KM == KM_POOLED;
  constexpr bool SPLIT = POOLED && ES == 2;
  constexpr int KRB = D * ES, KCPR = KRB / 16;   // K tile row: bytes, 16-byte chunks
  constexpr int VRB = BN * ES, VCPR = VRB / 16;  // V^T tile row
  constexpr int KT = BN * KRB, VT = D * VRB;
  constexpr int NBUF = ES == 2 ? 2 : 1;
  constexpr int STAGE = KT * (SPLIT ? 2 : 1) + VT;
  constexpr int NKC = BN * KCPR / 256;           // K chunks per thread per tile
  constexpr int DPT = D / 16;                    // V elements per key per thread
  constexpr int VW = DPT * ES / 4;               // 32-bit words per key per thread
  constexpr int NT = D / 32;                     // 32-wide output tiles over d

  __shared__ __attribute__((aligned(16))) char smem[NBUF * STAGE];
  __shared__ __attribute__((aligned(16))) float sbias[NBUF][BN];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int lid = xcd_remap(blockIdx.x, a.n_wg);
  const int bh = lid / a.tiles_per_head;
  const int rt = lid - bh * a.tiles_per_head;

  // ---- this lane's query row
  const long long vrow = (long long)rt * BM + w * 32 + l32;
  int qrow;
  if constexpr (RM == RM_IDENTITY) qrow = vrow < a.Ns ? (int)vrow : -1;
  else qrow = route_row(a.q_list + (long long)bh * a.q_k, a.q_k, a.b, a.nb_s, a.Ns, vrow);

  Op qB[D / 16];
  {
    const T* qp = (const T*)a.Q + rm_head(a.rmq, bh) + (long long)(qrow < 0 ? 0 : qrow) * a.rmq.sn + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (qrow >= 0) qB[s] = *(const Op*)(qp + 16 * s);
      else qB[s] = Op{};
    }
  }

  // ---- key range
  int n_keys, n_valid;
  if constexpr (KM == KM_DENSE) {
    n_keys = n_valid = a.Nk;
  } else if constexpr (KM == KM_GATHER) {
    n_keys = a.Ns + (int)a.ctx_tok;
    const bool tail_kept = a.kc > 0 && a.kept[(long long)bh * a.kc + a.kc - 1] == a.nb_c - 1;
    n_valid = n_keys - (tail_kept ? a.b - a.tail_c : 0);
  } else {
    n_keys = n_valid = a.mk_pad;
  }
  const int ntiles = (n_keys + BN - 1) / BN;

  const char* Kg;
  const char* Vg;
  const char* Klo = nullptr;
  long long krs = KRB, vrs = KRB;   // bytes between key rows, value rows
  if constexpr (POOLED) {
    Kg = (const char*)a.pkhi + (long long)bh * a.mk_pad * KRB;
    Vg = (const char*)a.pv + (long long)bh * a.mk_pad * KRB;
    if constexpr (SPLIT) Klo = (const char*)a.pklo + (long long)bh * a.mk_pad * KRB;
  } else {
    Kg = (const char*)a.K + rm_head(a.rmk, bh) * ES;
    Vg = (const char*)a.V + rm_head(a.rmv, bh) * ES;
    krs = a.rmk.sn * ES;
    vrs = a.rmv.sn * ES;
  }
  const int* crow = KM == KM_GATHER ? a.ctx_rows + (long long)bh * a.ctx_tok : nullptr;

  // source row of virtual key t, -1 if it is padding
  auto key_row = [&](int t) -> int {
    if (t >= n_valid) return -1;
    if constexpr (KM == KM_GATHER) return t < a.Ns ? t : crow[t - a.Ns];
    return t;
  };

  // ---- staged tile registers
  uint4 kreg[NKC];
  uint4 kreg_lo[SPLIT ? NKC : 1];
  uint32_t vreg[4][VW];
  float breg = 0.f;
  const int vdc = tid & 15, vkg = tid >> 4;   // V: d-group, 4-key group

  auto load_tile = [&](int tile) {
    const int t0 = tile * BN;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int q = tid + 256 * i;
      const int kr = q / KCPR, c = q % KCPR;
      const int row = key_row(t0 + kr);
      if (row >= 0) {
        kreg[i] = *(const uint4*)(Kg + (long long)row * krs + c * 16);
        if constexpr (SPLIT) kreg_lo[i] = *(const uint4*)(Klo + (long long)row * krs + c * 16);
      } else {
        kreg[i] = uint4{0, 0, 0, 0};
        if constexpr (SPLIT) kreg_lo[i] = uint4{0, 0, 0, 0};
      }
    }
if constexpr (WO) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = key_row(t0 + 4 * vkg + i);
        const char* src = Vg + (long long)(row < 0 ? 0 : row) * vrs + vdc * DPT * ES;
        if constexpr (VW == 2) {
          uint2 v = uint2{0, 0};
          if (row >= 0) v = *(const uint2*)src;
          vreg[i][0] = v.x; vreg[i][1] = v.y;
        } else {
#pragma unroll
          for (int u = 0; u < VW; u += 4) {
            uint4 v = uint4{0, 0, 0, 0};
            if (row >= 0) v = *(const uint4*)(src + 4 * u);
            vreg[i][u] = v.x; vreg[i][u + 1] = v.y; vreg[i][u + 2] = v.z; vreg[i][u + 3] = v.w;
          }
        }
      }
    }
    if constexpr (POOLED) {
      if (tid < BN) breg = a.pbias[(long long)bh * a.mk_pad + t0 + tid];
    }
  };

  auto store_tile = [&](int buf) {
    char* Ks = smem + buf * STAGE;
    char* Ks_lo = Ks + KT;
    char* Vs = Ks + KT * (SPLIT ? 2 : 1);
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int q = tid + 256 * i;
      const int kr = q / KCPR, c = q % KCPR;
      const int off = kr * KRB + swz(c, kr, KCPR) * 16;
      *(uint4*)(Ks + off) = kreg[i];
      if constexpr (SPLIT) *(uint4*)(Ks_lo + off) = kreg_lo[i];
    }
    // V^T: row d, 64 keys; key group g4 of each 16-key group sits at
    // position group {0,2,1,3}[g4] (the order of the P^T operand)
    if constexpr (WO) {
    const int g4 = vkg & 3;
    const int pos = 16 * (vkg >> 2) + 4 * (g4 == 1 ? 2 : (g4 == 2 ? 1 : g4));
    const int byte = pos * ES;
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
      const int d = vdc * DPT + j;
      const int off = d * VRB + swz(byte / 16, d, VCPR) * 16 + (byte & 15);
      if constexpr (ES == 2) {
        const int wd = j >> 1, sh = (j & 1) * 16;
        const uint32_t e0 = (vreg[0][wd] >> sh) & 0xffffu, e1 = (vreg[1][wd] >> sh) & 0xffffu;
        const uint32_t e2 = (vreg[2][wd] >> sh) & 0xffffu, e3 = (vreg[3][wd] >> sh) & 0xffffu;
        *(uint2*)(Vs + off) = uint2{e0 | (e1 << 16), e2 | (e3 << 16)};
      } else {
        *(uint4*)(Vs + off) = uint4{vreg[0][j], vreg[1][j], vreg[2][j], vreg[3][j]};
      }
    }
    }
    if constexpr (POOLED) {
      if (tid < BN) sbias[buf][tid] = breg;
    }
  };

  // 8 contraction elements [elem, elem+8) of row `row` of a swizzled tile
  auto lds_op = [&](const char* base, int row, int rb, int cpr, int elem) -> Op {
    const int byte = elem * ES;
    if constexpr (ES == 2) {
      return *(const Op*)(base + row * rb + swz(byte >> 4, row, cpr) * 16);
    } else {
      const f32x4 lo = *(const f32x4*)(base + row * rb + swz(byte >> 4, row, cpr) * 16);
      const f32x4 hi = *(const f32x4*)(base + row * rb + swz((byte >> 4) + 1, row, cpr) * 16);
      Op r;
      r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
      r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
      return r;
    }
  };

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = a.scale_log2;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  int cur = 0;
  for (int tile = 0; tile < ntiles; ++tile) {
    const bool has_next = tile + 1 < ntiles;
    if (has_next) load_tile(tile + 1);

    const char* Ks = smem + cur * STAGE;
    const char* Ks_lo = Ks + KT;
    const char* Vs = Ks + KT * (SPLIT ? 2 : 1);

    // S^T = K Q^T: lane holds query l32, keys 32*ti + 8*(r/4) + 4*h + r%4
    f32x16 S[2];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      S[ti] = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const Op kA = lds_op(Ks, 32 * ti + l32, KRB, KCPR, 16 * s + 8 * h);
        S[ti] = mma32(kA, qB[s], S[ti]);
        if constexpr (SPLIT) {
          const Op kL = lds_op(Ks_lo, 32 * ti + l32, KRB, KCPR, 16 * s + 8 * h);
          S[ti] = mma32(kL, qB[s], S[ti]);
        }
      }
    }

    // online softmax (exp2 domain)
    float mx = -INFINITY;
    if constexpr (POOLED) {
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 bb = *(const f32x4*)&sbias[cur][32 * ti + 8 * g + 4 * h];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = fmaf(S[ti][4 * g + e], sc, bb[e]);
            S[ti][4 * g + e] = x;
            mx = fmaxf(mx, x);
          }
        }
    } else {
      if (tile * BN + BN > n_valid) {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = tile * BN + 32 * ti + 8 * (r >> 2) + 4 * h + (r & 3);
            if (t >= n_valid) S[ti][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[ti][r]);
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float alpha, msub;
    if constexpr (POOLED) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      msub = m_new;
    } else {
      alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sc);
      msub = m_new * sc;
    }
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p;
        if constexpr (POOLED) p = __builtin_amdgcn_exp2f(S[ti][r] - msub);
        else p = __builtin_amdgcn_exp2f(fmaf(S[ti][r], sc, -msub));
        S[ti][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;

    if constexpr (WO) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
      // O^T += V^T P^T over 4 k-steps of 16 keys
      Op pB[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = S[s >> 1][8 * (s & 1) + j];
        make_operand(pv, pB[s]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const Op vA = lds_op(Vs, 32 * t + l32, VRB, VCPR, 16 * s + 8 * h);
          acc[t] = mma32(vA, pB[s], acc[t]);
        }
    }

    if (has_next) {
      if constexpr (NBUF == 1) __syncthreads();
      store_tile(cur ^ (NBUF - 1));
    }
    __syncthreads();
    cur ^= (NBUF - 1);
  }

  const float l_tot = l_run + wave_shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qrow >= 0) {
    if constexpr (WO) {
      T* op = (T*)a.O + rm_head(a.rmo, bh) + (long long)qrow * a.rmo.sn;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * t + 8 * g + 4 * h;
          const float o0 = acc[t][4 * g] * inv, o1 = acc[t][4 * g + 1] * inv;
          const float o2 = acc[t][4 * g + 2] * inv, o3 = acc[t][4 * g + 3] * inv;
          if constexpr (ES == 2) *(uint2*)(op + d0) = uint2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          else *(float4*)(op + d0) = float4{o0, o1, o2, o3};
        }
    }
    if constexpr (WP) {
      if (h == 0) a.peak[(long long)bh * a.Ns + qrow] = inv;
    }
  }
}

// ---------------------------------------------------------------------------

static AttnArgs attn_args(const Layout& L, const Bufs& B) {
  AttnArgs a = {};
  a.Q = B.Q; a.O = B.O; a.K = B.K; a.V = B.V;
  a.rmq = L.q; a.rmo = L.o; a.rmk = L.k; a.rmv = L.v;
  a.Ns = L.Ns; a.Nk = L.Nk;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)L.d));
  if (B.ws) {
    a.ctx_rows = (const int*)(B.ws + L.off_ctxrows);
    a.kept = (const int*)(B.ws + L.off_kept);
    a.pkhi = B.ws + L.off_pkhi;
    a.pklo = (const bf16_t*)(B.ws + L.off_pklo);
    a.pv = B.ws + L.off_pv;
    a.pbias = (const float*)(B.ws + L.off_pbias);
    a.peak = (float*)(B.ws + L.off_peak);
  }
  a.ctx_tok = L.ctx_tok;
  a.kc = L.kc; a.nb_c = L.nb_c; a.b = L.b; a.tail_c = L.tail_c;
  a.mk_pad = L.mk_pad;
  a.nb_s = L.nb_s;
  return a;
}

template <typename T, int D, int KM, int RM, bool WO, bool WP>
static hipError_t launch_attn_t(AttnArgs a, long long n_rows, long long BH, hipStream_t s) {
  a.n_rows = n_rows;
  a.tiles_per_head = (int)((n_rows + 127) / 128);
  const long long nwg = (long long)a.tiles_per_head * BH;
  if (nwg == 0) return hipSuccess;
  a.n_wg = (int)nwg;
  hipLaunchKernelGGL((isa_attn_kernel<T, D, KM, RM, WO, WP>), dim3((unsigned)nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t pooled_t(const Layout& L, const Bufs& B, int mode, hipStream_t s) {
  AttnArgs a = attn_args(L, B);
  if (mode == 0) return launch_attn_t<T, D, KM_POOLED, RM_IDENTITY, true, true>(a, L.Ns, L.BH, s);
  if (mode == 1) return launch_attn_t<T, D, KM_POOLED, RM_IDENTITY, false, true>(a, L.Ns, L.BH, s);
  a.q_list = (const int*)(B.ws + L.off_taylq);
  a.q_k = L.nb_s - L.kq;
  return launch_attn_t<T, D, KM_POOLED, RM_TABLE, true, false>(a, L.taylor_rows, L.BH, s);
}

template <typename T, int D>
static hipError_t full_t(const Layout& L, const Bufs& B, bool dense, hipStream_t s) {
  AttnArgs a = attn_args(L, B);
  if (dense) return launch_attn_t<T, D, KM_DENSE, RM_IDENTITY, true, false>(a, L.Ns, L.BH, s);
  a.q_list = (const int*)(B.ws + L.off_fullq);
  a.q_k = L.kq;
  return launch_attn_t<T, D, KM_GATHER, RM_TABLE, true, false>(a, L.full_rows, L.BH, s);
}

hipError_t launch_pooled_attention(const Layout& L, const Bufs& B, int mode, hipStream_t s) {
  if (L.es == 2) {
    const FlashWhat w = mode == 0 ? FlashWhat::kSharpTaylor : (mode == 1 ? FlashWhat::kSharp : FlashWhat::kTaylor);
    return launch_flash(L, B, w, s);
  }
  return L.d == 128 ? pooled_t<float, 128>(L, B, mode, s) : pooled_t<float, 64>(L, B, mode, s);
}

hipError_t launch_full_attention(const Layout& L, const Bufs& B, bool dense, hipStream_t s) {
  if (L.es == 2) return launch_flash(L, B, dense ? FlashWhat::kDense : FlashWhat::kFull, s);
  return L.d == 128 ? full_t<float, 128>(L, B, dense, s) : full_t<float, 64>(L, B, dense, s);
}

hipError_t launch_full_merge(const Layout& L, const Bufs& B, hipStream_t s) {
  if (L.es == 2) return launch_flash(L, B, FlashWhat::kFullMerge, s);
  return hipSuccess;
}

}  // namespace isa
