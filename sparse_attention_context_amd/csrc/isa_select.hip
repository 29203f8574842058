// Top-k selection, compaction and packing of the kept key set.
//
// ISA selects twice (Lightning Unified Video Editing via In-Context Sparse
// Attention, English abstract): which context blocks survive the pruning, and
// which query blocks, the sharpest, take the exact route.  Both keep the k
// highest scores.  The
// order is total: score descending, then index ascending, so ties go to the
// lower index.  Lists are emitted in ascending index order.
//
// One workgroup (4 waves) per (batch, head).  Scores are fp64 mapped to
// order-preserving 64-bit keys, so the selection itself is integer work:
//   n <= kRankMax: each wave sorts 128 (key, index) pairs in registers under
//                  the total order above (a bitonic network, partners
//                  exchanged by lane shuffles); a pair's rank is its
//                  position in its wave's run plus, for each other run, the
//                  number of pairs ahead of it (a binary search); the pairs
//                  of rank < k are selected;
//   n <= kSortMax: bitonic sort of (key, index) pairs in LDS under the total
//                  order above; the first k sorted positions are selected;
//   larger n:      MSB-first radix select, 8 passes of 8 bits with an LDS
//                  histogram, finds the k-th key T and how many keys equal
//                  to T are still needed.
// Compaction walks the indices in 256-wide chunks; a ballot + popcount
// prefix inside each wave and the wave totals give every element its slot.
#include "isa_device.h"
#include "isa_kernels.h"

namespace isa {

constexpr int kSortMax = 2048;
constexpr int kRankMax = 512;   // 4 waves x 64 lanes x 2 pairs

// (ka, ia) comes before (kb, ib): key descending, then index ascending
__device__ __forceinline__ bool first_before(uint64_t ka, int ia, uint64_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const unsigned lo = (unsigned)__shfl_xor((int)(unsigned)v, m, 64);
  const unsigned hi = (unsigned)__shfl_xor((int)(unsigned)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

struct SelectSmem {
  uint64_t keys[kSortMax];
  int idx[kSortMax];
  unsigned char chosen[kSortMax];
  int hist[256];
  int wtot[4];
  int wtot2[4];
  int digit;
  int above;
};

// Exclusive prefix count of `f` over the workgroup (thread order); *total
// gets the workgroup sum.  Contains barriers: call from every thread.
__device__ __forceinline__ int block_prefix(bool f, int* wtot, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t bal = __ballot(f);
  const int pre = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wtot[w] = __popcll(bal);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    off += i < w ? wtot[i] : 0;
    tot += wtot[i];
  }
  __syncthreads();
  *total = tot;
  return off + pre;
}

// Inclusive prefix sum of v over the workgroup (thread order).
__device__ __forceinline__ int block_inclusive_sum(int v, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) off += i < w ? wtot[i] : 0;
  __syncthreads();
  return v + off;
}

// Selects the k best of sc[0..n) and writes them ascending to sel[0..k);
// when rest is non-null the others go ascending to rest[0..n-k).
__device__ void select_topk(const double* sc, int n, int k, int* sel, int* rest, SelectSmem& sm) {
  const int tid = threadIdx.x;
  int mode;  // 0: none, 1: all, 2: sort, 3: radix, 4: rank
  if (k <= 0) mode = 0;
  else if (k >= n) mode = 1;
  else if (n <= kRankMax) mode = 4;
  else if (n <= kSortMax) mode = 2;
  else mode = 3;

  uint64_t T = 0;
  int need = 0;
  if (mode == 4) {
    // wave wv holds pairs 128 wv + 64 r + lane (r = 0, 1); padding pairs come last
    const int lane = tid & 63, wv = tid >> 6;
    uint64_t key[2];
    int id[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int e = 128 * wv + 64 * r + lane;
      key[r] = e < n ? order_key(sc[e]) : 0ull;
      id[r] = e < n ? e : 0x7fffffff;
    }
    for (int i = tid; i < n; i += 256) sm.chosen[i] = 0;
    // bitonic network over run position p = 64 r + lane: the run of length
    // `size` holding p is sorted first-to-last when (p & size) == 0
#pragma unroll
    for (int size = 2; size <= 128; size <<= 1) {
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        if (stride == 64) {   // (size 128: the whole run in one direction)
          if (first_before(key[1], id[1], key[0], id[0])) {
            const uint64_t tk = key[0];
            const int ti = id[0];
            key[0] = key[1]; id[0] = id[1];
            key[1] = tk; id[1] = ti;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const uint64_t pk = shfl_xor_u64(key[r], stride);
            const int pi = __shfl_xor(id[r], stride, 64);
            // the lower position of a pair keeps the pair's first entry in a
            // first-to-last run, its last entry otherwise
            const bool keep_first = ((lane & stride) == 0) == (((64 * r + lane) & size) == 0);
            if (first_before(pk, pi, key[r], id[r]) == keep_first) {
              key[r] = pk;
              id[r] = pi;
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      sm.keys[128 * wv + 64 * r + lane] = key[r];
      sm.idx[128 * wv + 64 * r + lane] = id[r];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (id[r] < n) {
        // pairs ahead of this one in each other run: the three searches interleaved
        int lo[3] = {0, 0, 0}, hi[3] = {128, 128, 128};
#pragma unroll
        for (int it = 0; it < 8; ++it) {
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            const int w2 = q + (q >= wv ? 1 : 0);
            if (lo[q] < hi[q]) {
              const int mid = (lo[q] + hi[q]) >> 1;
              if (first_before(sm.keys[128 * w2 + mid], sm.idx[128 * w2 + mid], key[r], id[r])) lo[q] = mid + 1;
              else hi[q] = mid;
            }
          }
        }
        if (64 * r + lane + lo[0] + lo[1] + lo[2] < k) sm.chosen[id[r]] = 1;
      }
    }
    __syncthreads();
  } else if (mode == 2) {
    // bitonic sort, descending by (key, then lower index first), padded to a
    // power of two with entries that sort last
    int np = 1;
    while (np < n) np <<= 1;
    for (int i = tid; i < np; i += 256) {
      sm.keys[i] = i < n ? order_key(sc[i]) : 0ull;
      sm.idx[i] = i < n ? i : 0x7fffffff;
      sm.chosen[i] = 0;
    }
    __syncthreads();
    for (int size = 2; size <= np; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (np >> 1); t += 256) {
          const int lo = 2 * t - (t & (stride - 1));
          const int hi = lo + stride;
          const bool desc = (lo & size) == 0;  // this run sorts descending
          const uint64_t ka = sm.keys[lo], kb = sm.keys[hi];
          const int ia = sm.idx[lo], ib = sm.idx[hi];
          const bool b_first = kb > ka || (kb == ka && ib < ia);
          if (b_first == desc) {
            sm.keys[lo] = kb; sm.keys[hi] = ka;
            sm.idx[lo] = ib; sm.idx[hi] = ia;
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < k; i += 256) sm.chosen[sm.idx[i]] = 1;
    __syncthreads();
  } else if (mode == 3) {
    uint64_t prefix = 0, mask = 0;
    need = k;
    for (int shift = 56; shift >= 0; shift -= 8) {
      sm.hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += 256) {
        const uint64_t key = order_key(sc[i]);
        if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255], 1);
      }
      __syncthreads();
      // suffix sums: thread t owns digit 255 - t
      const int dg = 255 - tid;
      const int cnt = sm.hist[dg];
      const int suf = block_inclusive_sum(cnt, sm.wtot);  // keys with digit >= dg
      if (suf >= need && suf - cnt < need) {
        sm.digit = dg;
        sm.above = suf - cnt;
      }
      __syncthreads();
      prefix |= (uint64_t)sm.digit << shift;
      mask |= 0xffull << shift;
      need -= sm.above;
      __syncthreads();
    }
    T = prefix;
  }

  int base_sel = 0, base_eq = 0;
  for (int c0 = 0; c0 < n; c0 += 256) {
    const int i = c0 + tid;
    const bool valid = i < n;
    bool f = false;
    if (mode == 1) {
      f = valid;
    } else if (mode == 2 || mode == 4) {
      f = valid && sm.chosen[i];
    } else if (mode == 3) {
      const uint64_t key = valid ? order_key(sc[i]) : 0;
      const bool eq = valid && key == T;
      int eq_tot;
      const int eq_pos = base_eq + block_prefix(eq, sm.wtot2, &eq_tot);
      base_eq += eq_tot;
      f = valid && (key > T || (eq && eq_pos < need));
    }
    int tot;
    const int pos = block_prefix(f, sm.wtot, &tot);
    if (valid) {
      const int ps = base_sel + pos, pr = i - ps;
      if (f) {
        if (ps < k) sel[ps] = i;
      } else if (rest && pr < n - k) {
        rest[pr] = i;
      }
    }
    base_sel += tot;
  }
}

struct SelArgs {
  const double* salp;
  double* sal;
  int* kept;
  int* ctx_rows;
  const float* peak;
  double* sh;
  int* full_q;
  int* taylor_q;
  int* key_rows;
  int Ns, Nc, b, nb_s, nb_c, kc, kq, sal_tiles, tail_s, n_keytab;
};

__global__ __launch_bounds__(256) void isa_select_ctx_kernel(SelArgs a) {
  __shared__ SelectSmem sm;
  const long long bh = blockIdx.x;
  const int tid = threadIdx.x;
  double* sal = a.sal + bh * a.nb_c;
  const double* part = a.salp + bh * (long long)a.sal_tiles * a.nb_c;
  for (int c = tid; c < a.nb_c; c += 256) {
    // the partials of 8 tiles are loaded before they are added (in tile order)
    double s = 0.0;
    int t = 0;
    for (; t + 8 <= a.sal_tiles; t += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(long long)(t + u) * a.nb_c + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; t < a.sal_tiles; ++t) s += part[(long long)t * a.nb_c + c];
    sal[c] = s;
  }
  __syncthreads();
  int* kept = a.kept + bh * a.kc;
  select_topk(sal, a.nb_c, a.kc, kept, nullptr, sm);
  __syncthreads();
  // full-route context key rows: kept block kb covers rows Ns + kb*b + [0, b),
  // -1 past the end of a short last block
  // (the kept list is staged through LDS 256 entries at a time, so the
  // loop below issues no dependent global loads)
  const int ntok = a.kc * a.b;
  int* rows = a.ctx_rows + bh * ntok;
  const unsigned ub = (unsigned)a.b;
  for (int k0 = 0; k0 < a.kc; k0 += 256) {
    const int nk = min(256, a.kc - k0);
    if (tid < nk) sm.idx[tid] = kept[k0 + tid];
    __syncthreads();
    const int t0 = k0 * a.b, t1 = (k0 + nk) * a.b;
    for (int t = t0 + tid; t < t1; t += 256) {
      const unsigned i = (unsigned)t / ub;
      const int kb = sm.idx[i - k0];
      const int r = kb * a.b + (int)((unsigned)t - i * ub);
      rows[t] = (kb >= 0 && kb < a.nb_c && r < a.Nc) ? a.Ns + r : -1;
    }
    __syncthreads();
  }
}

// Workgroups (bh, y > 0) of the query selection write chunk y - 1 of the
// head's full-route key-row table, beside the selection of workgroup (bh, 0):
// the K/V row of every key of the route, four per store -- the source rows,
// then the context rows (a short last block's -1 and the padding up to whole
// tiles read row 0; the attention masks those keys).
constexpr int kKeyTabChunk = 256 * 4 * 8;

__global__ __launch_bounds__(256) void isa_select_q_kernel(SelArgs a) {
  __shared__ SelectSmem sm;
  const long long bh = blockIdx.x;
  const int tid = threadIdx.x;
  if (blockIdx.y > 0) {
    const int ntok = a.kc * a.b;
    const int* crow = a.ctx_rows + bh * ntok;
    int4* tab = (int4*)(a.key_rows + bh * a.n_keytab);
    const int q0 = (int)(blockIdx.y - 1) * (kKeyTabChunk / 4);
    const int q1 = min(q0 + kKeyTabChunk / 4, a.n_keytab / 4);
    for (int q = q0 + tid; q < q1; q += 256) {
      int v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = 4 * q + u;
        v[u] = t < a.Ns ? t : (t - a.Ns < ntok ? max(crow[t - a.Ns], 0) : 0);
      }
      tab[q] = int4{v[0], v[1], v[2], v[3]};
    }
    return;
  }
  double* sh = a.sh + bh * a.nb_s;
  const float* pk = a.peak + bh * a.Ns;
  // block means of the per-row peaks, rows added in order; the rows of a
  // block are fetched 32 at a time with independent loads
  for (int i = tid; i < a.nb_s; i += 256) {
    const int r0 = i * a.b;
    const int n = min(a.b, a.Ns - r0);
    double s = 0.0;
    int r = 0;
    for (; r + 32 <= n; r += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = pk[r0 + r + u];
#pragma unroll
      for (int u = 0; u < 32; ++u) s += (double)v[u];
    }
    for (; r < n; ++r) s += (double)pk[r0 + r];
    sh[i] = s / n;
  }
  __syncthreads();
  int* fq = a.full_q + bh * a.kq;
  int* tq = a.taylor_q + bh * (a.nb_s - a.kq);
  select_topk(sh, a.nb_s, a.kq, fq, tq, sm);
}

static SelArgs sel_args(const Layout& L, const Bufs& B) {
  SelArgs a;
  a.salp = (const double*)(B.ws + L.off_salp);
  a.sal = (double*)(B.ws + L.off_sal);
  a.kept = (int*)(B.ws + L.off_kept);
  a.ctx_rows = (int*)(B.ws + L.off_ctxrows);
  a.peak = (const float*)(B.ws + L.off_peak);
  a.sh = (double*)(B.ws + L.off_sh);
  a.full_q = (int*)(B.ws + L.off_fullq);
  a.taylor_q = (int*)(B.ws + L.off_taylq);
  a.key_rows = (int*)(B.ws + L.off_keyrows);
  a.n_keytab = L.n_keytab;
  a.Ns = L.Ns; a.Nc = L.Nc; a.b = L.b; a.nb_s = L.nb_s; a.nb_c = L.nb_c;
  a.kc = L.kc; a.kq = L.kq; a.sal_tiles = L.sal_tiles; a.tail_s = L.tail_s;
  return a;
}

hipError_t launch_select_ctx(const Layout& L, const Bufs& B, hipStream_t s) {
  if (L.nb_c == 0) return hipSuccess;
  hipLaunchKernelGGL(isa_select_ctx_kernel, dim3((unsigned)L.BH), dim3(256), 0, s, sel_args(L, B));
  return hipGetLastError();
}

hipError_t launch_select_q(const Layout& L, const Bufs& B, hipStream_t s) {
  // the key-row table is needed by the full route only
  const unsigned chunks = L.kq > 0 ? (unsigned)((L.n_keytab + kKeyTabChunk - 1) / kKeyTabChunk) : 0u;
  hipLaunchKernelGGL(isa_select_q_kernel, dim3((unsigned)L.BH, 1u + chunks), dim3(256), 0, s, sel_args(L, B));
  return hipGetLastError();
}

}  // namespace isa
