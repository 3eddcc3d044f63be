// Token indexer scores and the vertical-slash estimate (bf16 matrix cores).
//
// IndexCache article, §长文本的算力困境: a light indexer scores every causal
// (query, key) pair, and its quadratic cost becomes the prefill bottleneck.
// Score of the synthetic workload: I[t,s] = sum_h w_h * ReLU(q[t,h] . k[s]).
// The contraction q[t,h] . k[s] is a dense GEMM per head; the ReLU sits
// between it and the sum over heads, so each head's tile is finished in
// registers (max, then FMA with w_h).  With 32 or 64 heads the heads lie on
// the matrix rows (k_indexer2); other head counts split the heads over eight
// waves that reduce their partial sums through LDS (k_indexer).
//
// "MInference 1.0" article, §方法介紹: vertical and slash indices come from
// the attention of the last queries to every key.  Pass 1 gathers per-chunk
// softmax statistics of the last 64 query rows; pass 2 recomputes the
// probabilities tile by tile and reduces them along columns (vertical score)
// and along diagonals (slash score, offset = query position - key).  The
// diagonal sums of each 64-key tile are written as partials and merged in a
// fixed order by a last kernel, so the result is deterministic.
//
// k_indexer2 and the vertical-slash passes stage 64-key K tiles in LDS by
// direct copies, shared by every wave of the workgroup (the indexer's query
// groups, or the query heads of one KV head), and feed them to
// v_mfma_f32_32x32x16_bf16; k_indexer reads its K rows into registers.
//
// The indexer's fused top-k (a sampled threshold, a pass that keeps only the
// keys reaching it, an exact select over those) lives here too.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "select_util.h"

namespace sa {
namespace {

// ================================================================ indexer
// max(x, 0) as one integer max on the bit pattern: every negative float
// (including -0) is a negative int32; finite inputs only (products of bf16).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// The integer ReLU above turns a NaN product with its sign bit set into 0, so
// a NaN in the indexer's inputs need not reach its scores.  When the caller
// asks for the flag, this pass sets bit 0 if any element of q, k (bf16, 8 per
// 16-byte load) or the weights is NaN or infinite.
__global__ __launch_bounds__(256) void k_idx_scan_inputs(const uint16_t* __restrict__ q, int64_t nq8,
                                                         const uint16_t* __restrict__ k, int64_t nk8,
                                                         const float* __restrict__ w, int nw, int32_t* err) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  auto bad2 = [](uint32_t x) { return (x & 0x7f80u) == 0x7f80u || (x & 0x7f800000u) == 0x7f800000u; };
  bool bad = false;
  for (int64_t i = t0; i < nq8 + nk8; i += stride) {
    const u32x4 v = ldg16(i < nq8 ? q + 8 * i : k + 8 * (i - nq8));
    bad |= bad2(v[0]) || bad2(v[1]) || bad2(v[2]) || bad2(v[3]);
  }
  for (int64_t i = t0; i < nw; i += stride) bad |= nonfinite(w[i]);
  flag_nonfinite(err, bad);
}

hipError_t scan_indexer_inputs(const uint16_t* q, const uint16_t* k, const float* w, int T, int hi, int64_t nk,
                               int32_t* err, hipStream_t stream) {
  if (err == nullptr) return hipSuccess;
  const int64_t nq8 = (int64_t)T * hi * 64 / 8, nk8 = nk * 64 / 8;
  const int64_t blocks = std::min<int64_t>(2048, (nq8 + nk8 + 255) / 256 + 1);
  hipLaunchKernelGGL(k_idx_scan_inputs, dim3((unsigned)blocks), dim3(256), 0, stream, q, nq8, k, nk8, w, hi, err);
  return hipGetLastError();
}

constexpr int kIdxWaves = 8;
constexpr int kIdxD = 64;
constexpr int kIdxChunk = 8192;  // keys per workgroup

template <int HPW>
__global__ __launch_bounds__(64 * kIdxWaves) void k_indexer(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                            const float* __restrict__ w, int T, int Hi, int64_t Nk,
                                                            int64_t pos0, float* __restrict__ out,
                                                            int32_t* __restrict__ err) {
  __shared__ float red[kIdxWaves][64 * 33];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int nchunk = (int)((Nk + kIdxChunk - 1) / kIdxChunk);
  const int tq = blockIdx.x / nchunk, ck = blockIdx.x % nchunk;
  const int t0 = tq * 32;
  const int64_t c0 = (int64_t)ck * kIdxChunk, c1 = std::min(Nk, c0 + kIdxChunk);
  const int tl = std::min(t0 + l32, T - 1);
  // Q^T for this wave's heads: query tl, dims 32hf + 8s .. +7 at step s
  bf16x8 qv[HPW][4];
  float wh[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int h = wv * HPW + j;
    wh[j] = w[h];
    const uint16_t* qr = q + ((int64_t)tl * Hi + h) * kIdxD + 32 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[j][s] = as_bf16x8(ldg16(qr + 8 * s));
  }
  const int64_t lim_max = pos0 + std::min(t0 + 31, T - 1);  // largest causal key of the tile's queries
  const int tid = threadIdx.x;
  bool bad = false;
  for (int64_t s0 = c0; s0 < c1; s0 += 64) {
    const bool live = s0 <= lim_max;
    if (live) {
      bf16x8 ka[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int64_t row = std::min(s0 + 32 * mt + l32, Nk - 1);
        const uint16_t* kr = k + row * kIdxD + 32 * hf;
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[mt][s] = as_bf16x8(ldg16(kr + 8 * s));
      }
      float sum[32];
#pragma unroll
      for (int r = 0; r < 32; ++r) sum[r] = 0.f;
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        f32x16 a0, a1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          a0[r] = 0.f;
          a1[r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          a0 = mfma32x32x16(ka[0][s], qv[j][s], a0);
          a1 = mfma32x32x16(ka[1][s], qv[j][s], a1);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sum[r] = fmaf(wh[j], relu_bits(a0[r]), sum[r]);
          sum[16 + r] = fmaf(wh[j], relu_bits(a1[r]), sum[16 + r]);
        }
      }
      // element (mt, r) is key 32mt + 8(r/4) + 4hf + r%4 of the tile, query l32
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int key = 32 * (r / 16) + 8 * ((r % 16) / 4) + 4 * hf + (r % 4);
        red[wv][key * 33 + l32] = sum[r];
      }
    }
    __syncthreads();
    // fixed-order sum over the waves; thread -> (query, 4 consecutive keys)
    for (int e = tid; e < 32 * 16; e += 64 * kIdxWaves) {
      const int qq = e / 16, kq = e % 16;
      const int t = t0 + qq;
      if (t < T) {
        const int64_t lim = pos0 + t;
        f32x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 4 * kq + i;
          float acc = 0.f;
          if (live) {
#pragma unroll
            for (int ww = 0; ww < kIdxWaves; ++ww) acc += red[ww][key * 33 + qq];
          }
          v4[i] = (s0 + key > lim) ? -INFINITY : acc;
          bad |= s0 + key <= lim && s0 + key < c1 && nonfinite(acc);
        }
        const int64_t s = s0 + 4 * kq;
        float* op = out + (int64_t)t * Nk + s;
        if (s + 3 < c1) {
          *reinterpret_cast<f32x4*>(op) = v4;
        } else {
          for (int i = 0; i < 4 && s + i < c1; ++i) op[i] = v4[i];
        }
      }
    }
    __syncthreads();
  }
  flag_nonfinite(err, bad);
}

// Heads on the matrix rows.  For a query t the product Q_t . K^T puts the 32
// heads of a head group on the rows of v_mfma_f32_32x32x16_bf16 and 32 keys on
// its columns, so each lane holds 16 heads of one key: the ReLU and the
// weighted sum over heads are 16 in-register FMAs and one exchange with the
// lane holding the other 16 heads (v_permlane32_swap, no LDS round trip).  A
// workgroup (4 waves x 4 queries, two workgroups per CU) walks its key range
// in tiles of 64 keys copied once into LDS (double-buffered) and shared by all
// waves; there is no cross-wave reduction.  Queries per wave: 4 with one head
// group, 3 with two (the query operands then fill 96 registers).  Within a
// tile the products of the next (key half, query, head group) unit run on the
// matrix cores while the VALU finishes the current one.
constexpr int kIdx2Waves = 4;
template <int HG>
constexpr int idx2_qpw() { return HG == 1 ? 4 : 3; }

// chunk c of row r of a 64 x 128-byte K tile sits at position c ^ ((r >> 1) & 7)
__device__ __forceinline__ int idx2_swz(int r, int c) { return r * 64 + 8 * (c ^ ((r >> 1) & 7)); }

// Candidate output of the indexer when the scores are not stored: for every
// query a threshold (-inf keeps every key), and per chunk of keys a run of
// slots at a fixed place in the query's row of the candidate buffer.
struct IdxCand {
  const float* thr;     // [T]
  int2* cand;           // [T, rs] (key, score bits), ascending keys within a chunk
  int32_t* segc;        // [T, nseg] keys kept per chunk (may exceed the slots)
  int32_t* err;         // bit 0: a NaN score; bit 1: a failed row
  int64_t rs;
  int nseg;
  int expect;           // expected kept keys of a full row
};

template <int HG, bool CAND>
__global__ __launch_bounds__(64 * kIdx2Waves, 2) void k_indexer2(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const float* __restrict__ w, int T, int Hi,
                                                               int64_t Nk, int kstride, int chunk, int64_t pos0,
                                                               float* __restrict__ out, IdxCand cd) {
  constexpr int kIdx2Qpw = idx2_qpw<HG>(), kIdx2Q = kIdx2Waves * kIdx2Qpw;
  __shared__ __attribute__((aligned(1024))) uint16_t Kt[2][64 * kIdxD];
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunk = (int)((Nk + chunk - 1) / chunk);
  const int tq = blockIdx.x / nchunk, ck = blockIdx.x % nchunk;
  const int t0 = tq * kIdx2Q;
  const int64_t c0 = (int64_t)ck * chunk, c1 = std::min(Nk, c0 + chunk);
  // column c scores key c * kstride; the largest causal column of the queries
  const int64_t lim_max = (pos0 + std::min(t0 + kIdx2Q - 1, T - 1)) / kstride;
  // A operands: query t0 + 4wv + j, head 32g + l32, dims 16s + 8hf .. +7
  bf16x8 qa[kIdx2Qpw][HG][4];
#pragma unroll
  for (int j = 0; j < kIdx2Qpw; ++j) {
    const int t = std::min(t0 + kIdx2Qpw * wv + j, T - 1);
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      const uint16_t* qr = q + ((int64_t)t * Hi + 32 * g + l32) * kIdxD + 8 * hf;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) qa[j][g][s4] = as_bf16x8(ldg16(qr + 16 * s4));
    }
  }
  // weight of the head on accumulator row r: 32g + 8(r/4) + 4hf + r%4
  float wr[HG][16];
#pragma unroll
  for (int g = 0; g < HG; ++g)
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[g][r] = w[32 * g + 8 * (r / 4) + 4 * hf + (r % 4)];
  // candidate mode: per query its threshold, last causal key of the chunk,
  // slot run and running count
  float thr[kIdx2Qpw];
  int lim[kIdx2Qpw], nslot[kIdx2Qpw], found[kIdx2Qpw];
  int2* run[kIdx2Qpw];
  if constexpr (CAND) {
#pragma unroll
    for (int j = 0; j < kIdx2Qpw; ++j) {
      const int t = t0 + kIdx2Qpw * wv + j;
      const int64_t n = std::min(Nk, pos0 + t + 1);
      const bool any = t < T && c0 < n;
      thr[j] = any ? cd.thr[t] : 0.f;
      lim[j] = any ? (int)(std::min(n, c1) - 1) : -1;
      nslot[j] = any ? (int)idx_slots(n, ck, chunk, cd.expect) : 0;
      run[j] = cd.cand + (any ? (int64_t)t * cd.rs + ck * idx_slots(n, 0, chunk, cd.expect) : 0);
      found[j] = 0;
    }
  }
  drain_vmem();

  const int64_t s_end = std::min(c1, lim_max + 1);  // keys past every query's limit are only written
  const int ntile = s_end > c0 ? (int)((s_end - c0 + 63) / 64) : 0;
  // 1 KB copies (8 rows each), 8 / kIdx2Waves per wave: rows 8wq .. 8wq+7
  auto copy = [&](int tl, int buf) {
#pragma unroll
    for (int n = 0; n < 8 / kIdx2Waves; ++n) {
      const int wq = wv + n * kIdx2Waves;
      const int r = 8 * wq + lane / 8, c = lane % 8;
      const int64_t row = std::min(c0 + 64 * (int64_t)tl + r, Nk - 1) * kstride;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(&Kt[buf][0]) + (uint32_t)wq * 1024u);
      dma16(dst, k + row * kIdxD + 8 * (c ^ ((r >> 1) & 7)));
    }
  };
  if (ntile > 0) copy(0, 0);
  for (int tl = 0; tl < ntile; ++tl) {
    const int buf = tl & 1;
    wait_vmcnt<0>();
    __syncthreads();  // tile tl landed for every wave; buffer buf^1 is free
    if (tl + 1 < ntile) copy(tl + 1, buf ^ 1);
    const int64_t s0 = c0 + 64 * (int64_t)tl;
    // both 32-key halves of the tile; unit u = (half hv, query j, head group g)
    bf16x8 kb[2][4];
#pragma unroll
    for (int hv = 0; hv < 2; ++hv)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        kb[hv][s4] = as_bf16x8(*reinterpret_cast<const u32x4*>(&Kt[buf][idx2_swz(32 * hv + l32, 2 * s4 + hf)]));
    constexpr int UH = kIdx2Qpw * HG, U = 2 * UH;
    f32x16 acc[2];
    auto prod = [&](int u, f32x16& a) {
      const int hv = u / UH, j = (u / HG) % kIdx2Qpw, g = u % HG;
      a = mfma32x32x16(qa[j][g][0], kb[hv][0], f32x16{});
#pragma unroll
      for (int s4 = 1; s4 < 4; ++s4) a = mfma32x32x16(qa[j][g][s4], kb[hv][s4], a);
    };
    // the products of unit u+1 run on the matrix cores while the ReLU-weighted
    // sum of unit u runs on the VALU
    prod(0, acc[0]);
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int hv = u / UH, j = (u / HG) % kIdx2Qpw, g = u % HG;
      if (u + 1 < U) prod(u + 1, acc[(u + 1) & 1]);
#pragma unroll
      for (int r = 0; r < 16; ++r) sum = fmaf(wr[g][r], relu_bits(acc[u & 1][r]), sum);
      if (u + 1 < U) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
          __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);  // eight VALU
        }
      }
      if (g == HG - 1) {
        // lane l < 32 adds the partial sum of lane l + 32 (the other 16 heads)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
        const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int t = t0 + kIdx2Qpw * wv + j;
        const int64_t key = s0 + 32 * hv + l32;
        if constexpr (CAND) {
          // lanes 0..31 hold keys s0+32hv .. +31 in order: a ballot ranks
          // the kept ones, so every chunk's run is stored ascending.  A NaN
          // score is kept (the exact select reports it).
          const bool take = hf == 0 && (int)key <= lim[j] && !(tot < thr[j]);
          const uint64_t m = __ballot(take);
          if (take) {
            const int pos = found[j] + (int)__builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u);
            if (pos < nslot[j]) run[j][pos] = make_int2((int)key, __float_as_int(tot));
          }
          found[j] += __popcll(m);
        } else {
          if (hf == 0 && t < T && key < c1) {
            const bool causal = key * kstride <= pos0 + t;
            out[(int64_t)t * Nk + key] = causal ? tot : -INFINITY;
            flag_nonfinite(cd.err, causal && nonfinite(tot));
          }
        }
        sum = 0.f;
      }
    }
  }
  if constexpr (CAND) {
#pragma unroll
    for (int j = 0; j < kIdx2Qpw; ++j) {
      const int t = t0 + kIdx2Qpw * wv + j;
      if (lane == 0 && nslot[j] > 0) cd.segc[(int64_t)t * cd.nseg + ck] = found[j];
    }
  } else {
    // keys of the chunk beyond every query's causal limit
    for (int64_t sidx = std::max(c0, s_end) + lane; sidx < c1; sidx += 64)
#pragma unroll
      for (int j = 0; j < kIdx2Qpw; ++j) {
        const int t = t0 + kIdx2Qpw * wv + j;
        if (t < T) out[(int64_t)t * Nk + sidx] = -INFINITY;
      }
  }
}

// ---------------------------------------------------------------- indexer top-k
// The top k of a query's scores without the score matrix.  A row of at most
// kIdxSelCap keys keeps all of them.  For a longer row, a pass over every 16th
// key (kIdxStride) gives the query a threshold, the kIdxRank-th largest
// sampled score, which about 16 * kIdxRank = 4096 keys of the full row reach
// (relative spread ~1/sqrt(kIdxRank), so k <= 2048 lies 8 spreads below).
// The full pass keeps only the keys at or above the threshold; when at least k
// of them are kept, the row's top k are exactly the top k of the kept keys
// (every other key scores below the threshold, hence below the k-th kept
// one), and a radix select over them ends the row.
constexpr int kIdxStride = 16;
constexpr int kIdxRank = 256;
constexpr int kIdxExpect = kIdxStride * kIdxRank;  // kept keys expected in a long row
constexpr int kIdxSampleChunk = 1024;  // sampled keys per workgroup
constexpr int kIdxSelCap = 8192;       // kept keys a row may have in the exact select
constexpr int kIdxSelNT = 256;
constexpr int kIdxThrCap = 8192;       // sampled scores staged in LDS by the threshold kernel

// Threshold per query: -inf (every key) for a row of at most kIdxSelCap keys,
// else the kIdxRank-th largest of its causal sampled scores.  A NaN sample
// sets bit 0 of err.
__global__ __launch_bounds__(256) void k_idx_thresh(const float* __restrict__ smp, int64_t ns, int64_t Nk,
                                                    int64_t pos0, float* __restrict__ thr,
                                                    int32_t* __restrict__ err) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[4];
  __shared__ uint32_t shv[4];
  __shared__ uint32_t keys[kIdxThrCap];
  const int t = blockIdx.x;
  if (std::min(Nk, pos0 + t + 1) <= kIdxSelCap) {
    if (threadIdx.x == 0) thr[t] = -INFINITY;
    return;
  }
  // causal sampled keys: 16c <= pos0 + t; more than kIdxSelCap / 16 >= kIdxRank of them
  const int64_t n = std::min(ns, (pos0 + t) / kIdxStride + 1);
  const int m = kIdxRank;
  const float* row = smp + (int64_t)t * ns;
  bool nan_seen = false;
  const bool staged = n <= kIdxThrCap;
  // batches of 8 independent loads per thread keep the row's reads in flight
  for (int64_t b = 0; b < n; b += 256 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = b + u * 256 + threadIdx.x;
      v[u] = i < n ? row[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = b + u * 256 + threadIdx.x;
      if (i < n) {
        nan_seen |= is_nan(v[u]);
        if (staged) keys[i] = order_key(v[u]);
      }
    }
  }
  __syncthreads();
  if (nan_seen && err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(err), 1u);
  uint32_t kth;
  int64_t need;
  if (staged)
    radix_kth<256>([&](int64_t i) { return keys[i]; }, 0, n, m, hist, tmp, shv, kth, need);
  else
    radix_kth<256>([&](int64_t i) { return order_key(row[i]); }, 0, n, m, hist, tmp, shv, kth, need);
  // back from the order key to the float (the k-th key is never a NaN's
  // unless the row holds NaNs, which err reports)
  if (threadIdx.x == 0) thr[t] = __uint_as_float((kth & 0x80000000u) ? (kth ^ 0x80000000u) : ~kth);
}

// Exact top k of one query over its kept keys.  The chunks' runs are copied
// into LDS in chunk order, so the kept keys lie ascending; the k-th largest
// order key is found by radix select and one pass emits, ascending, every key
// above it and the lowest-index keys equal to it.  A row whose runs overflowed
// or that kept fewer than k keys gets cnt = -1, idx all -1 and bit 1 of err.
__global__ __launch_bounds__(kIdxSelNT) void k_idx_select(IdxCand cd, int64_t Nk, int64_t pos0, int chunk, int k,
                                                          int kmax, int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ cnt) {
  constexpr int NT = kIdxSelNT;
  __shared__ uint32_t sk[kIdxSelCap];
  __shared__ int32_t si[kIdxSelCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmp[NT / 64];
  __shared__ uint32_t shv[4];
  __shared__ int pre[NT + 1];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int64_t n = std::min(Nk, pos0 + t + 1);
  const int64_t kr = std::min<int64_t>(k, n);
  int32_t* out = idx + (int64_t)t * kmax;
  if (kr == n) {  // the row keeps every causal key
    for (int64_t j = tid; j < kmax; j += NT) out[j] = j < n ? (int32_t)j : -1;
    if (tid == 0) cnt[t] = (int32_t)n;
    return;
  }
  const int nch = (int)((n + chunk - 1) / chunk);
  const int64_t run = idx_slots(n, 0, chunk, cd.expect);
  const int2* src = cd.cand + (int64_t)t * cd.rs;
  int total = 0;
  bool bad = false, nan_seen = false;
  // chunks in groups of NT: thread c reads chunk c's count, a scan places the
  // runs, and every thread copies kept keys of any run (8 loads in flight)
  for (int g0 = 0; g0 < nch && !bad; g0 += NT) {
    const int c = g0 + tid;
    const int fc = c < nch ? cd.segc[(int64_t)t * cd.nseg + c] : 0;
    const bool over = c < nch && fc > idx_slots(n, c, chunk, cd.expect);
    uint32_t gtot;
    const uint32_t before = block_excl_scan<NT>((uint32_t)fc, tmp, gtot);
    pre[tid] = (int)before;
    if (tid == 0) pre[NT] = (int)gtot;
    if (__syncthreads_or(over) || total + (int64_t)gtot > kIdxSelCap) {
      bad = true;
      break;
    }
    const int ng = min(NT, nch - g0);
    for (int f0 = 0; f0 < (int)gtot; f0 += NT * 8) {
      int2 e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int f = f0 + u * NT + tid;
        e[u] = make_int2(0, 0);
        if (f < (int)gtot) {
          int lo = 0, hi = ng - 1;  // the run holding flat position f: last lo with pre[lo] <= f
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= f) lo = mid;
            else hi = mid - 1;
          }
          e[u] = src[(int64_t)(g0 + lo) * run + (f - pre[lo])];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int f = f0 + u * NT + tid;
        if (f < (int)gtot) {
          const float v = __int_as_float(e[u].y);
          nan_seen |= is_nan(v);
          sk[total + f] = order_key(v);
          si[total + f] = e[u].x;
        }
      }
    }
    total += (int)gtot;
    __syncthreads();  // pre[] is rewritten by the next group
  }
  if (__syncthreads_or(nan_seen) && tid == 0 && cd.err != nullptr)
    atomicOr(reinterpret_cast<unsigned int*>(cd.err), 1u);
  if (bad || total < kr) {
    for (int64_t j = tid; j < kmax; j += NT) out[j] = -1;
    if (tid == 0) {
      cnt[t] = -1;
      if (cd.err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(cd.err), 2u);
    }
    return;
  }
  __syncthreads();
  uint32_t kth;
  int64_t need;
  radix_kth<NT>([&](int64_t i) { return sk[i]; }, 0, total, kr, hist, tmp, shv, kth, need);
  // emission in LDS (= key) order, tiles of NT*4 kept keys
  uint32_t gt_run = 0u, eq_run = 0u;
  for (int b0 = 0; b0 < total; b0 += NT * 4) {
    const int i0 = b0 + tid * 4;
    uint32_t f[4];
    uint32_t c_gt = 0u, c_eq = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e;
      const uint32_t kk = i < total ? sk[i] : 0u;
      f[e] = i < total ? (kk > kth ? 1u : (kk == kth ? 2u : 0u)) : 0u;
      c_gt += f[e] == 1u;
      c_eq += f[e] == 2u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<NT>((c_eq << 16) | c_gt, tmp, tot);
    uint32_t g_before = gt_run + (ex & 0xffffu);
    uint32_t e_before = eq_run + (ex >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e;
      if (f[e] == 1u) {
        out[g_before + (uint32_t)min((int64_t)e_before, need)] = si[i];
        ++g_before;
      } else if (f[e] == 2u) {
        if ((int64_t)e_before < need) out[g_before + e_before] = si[i];
        ++e_before;
      }
    }
    gt_run += tot & 0xffffu;
    eq_run += tot >> 16;
  }
  for (int64_t j = kr + tid; j < kmax; j += NT) out[j] = -1;
  if (tid == 0) cnt[t] = (int32_t)kr;
}

// ================================================================ vertical-slash estimate
constexpr int kVsLast = 64;
constexpr int kVsTilesPerWg = 16;

// One workgroup per (batch, KV head, block of up to 4 of its query heads,
// chunk of 16 key tiles): the 64-key K tiles go into LDS once, by direct
// copies (double-buffered), and serve every listed query head of the KV head.
// Wave w takes query head slot w/2 and key half w%2 (32 keys) of each tile,
// for all 64 last queries of that head (two 32-query operand tiles kept in
// registers).  Lane (l32, hf) reads key row l32 of its half, dims 8hf + 16s ..
// +7 at step s, from LDS; the rows' 16-byte chunks sit XOR-swizzled so that
// eight consecutive rows read the same chunk from distinct banks.
constexpr int kVsWaves = 8;

template <int D>
__device__ __forceinline__ int vs_swz(int r, int c) {
  return D == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

// Compact output row of query head h of batch b (-1 when a head list leaves it out).
__device__ __forceinline__ int vs_row(const HeadList& hl, int hq, int b, int h) {
  if (hl.n == 0) return b * hq + h;
  for (int i = 0; i < hl.n; ++i)
    if (hl.h[i] == h) return b * hl.n + i;
  return -1;
}

// PASS 2 = false: per (row, chunk, query) running max and sum (log2 domain).
// PASS 2 = true: probabilities (exp2(s * sl2 - M') with M' = M + log2 L)
// reduced along the queries (column sums, final) and along the diagonals of
// each 64 x 64 tile (partials, merged by k_vs_slash).
template <int D, bool PASS2>
__global__ __launch_bounds__(64 * kVsWaves) void k_vs_pass(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                           int hq, int hkv, HeadList hl, int64_t N, float sl2,
                                                           int nchunk, int nhs, const float* __restrict__ ml,
                                                           float* __restrict__ stats, float* __restrict__ a_v,
                                                           float* __restrict__ dpart) {
  constexpr int NS = D / 16, CPR = D / 8;  // k-steps; 16-byte chunks per row
  constexpr int NB = PASS2 ? 2 : 3;  // K tile buffers: pass 1 copies two tiles ahead
  __shared__ __attribute__((aligned(1024))) uint16_t Kt[NB][64 * D];
  __shared__ __attribute__((aligned(16))) float Pl[PASS2 ? 4 : 1][64][kVsLast + 4];  // [head slot][key][query]
  __shared__ float st[4][2][kVsLast][2];             // pass 1: [head slot][key half][query](m, l)
  // pass 2: the chunk's column sums and diagonal partials, written out after
  // the loop so that no store sits in front of the per-tile copy wait
  __shared__ float av_s[PASS2 ? 4 : 1][PASS2 ? kVsTilesPerWg * 64 : 1];
  __shared__ float dp_s[PASS2 ? 4 : 1][PASS2 ? kVsTilesPerWg : 1][128];
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31, tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ck = blockIdx.x % nchunk, rest = blockIdx.x / nchunk;
  const int hs = rest % nhs, bg = rest / nhs;
  const int b = bg / hkv, g = bg % hkv;
  const int grp = hq / hkv;
  const int js = wv >> 1, kh = wv & 1;
  // rows of the four head slots (every thread, for the diagonal pass)
  int rows[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rows[j] = (4 * hs + j < grp) ? vs_row(hl, hq, b, g * grp + 4 * hs + j) : -1;
  const int row = rows[js];
  const bool active = row >= 0;
  const int h = g * grp + 4 * hs + js;
  const uint16_t* kb = k + ((int64_t)b * hkv + g) * N * D;
  const int64_t ntile = N / 64;
  const int64_t tb = (int64_t)ck * kVsTilesPerWg, te = std::min(ntile, tb + kVsTilesPerWg);
  const int nt = (int)(te - tb);
  // query operands: query 32qt + l32 of the last 64, dims 8hf + 16s .. +7
  bf16x8 qv[2][NS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const uint16_t* qr = q + (((int64_t)b * hq + (active ? h : 0)) * N + (N - kVsLast) + 32 * qt + l32) * D + 8 * hf;
#pragma unroll
    for (int s4 = 0; s4 < NS; ++s4) qv[qt][s4] = as_bf16x8(ldg16(qr + 16 * s4));
  }
  // pass 2: M' of the 16 queries this lane's accumulator rows hold per query tile
  float mq[2][16];
  if constexpr (PASS2) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 32 * qt + 8 * (r / 4) + 4 * hf + (r % 4);
        const float* mp = ml + ((int64_t)(active ? row : 0) * kVsLast + qi) * 2;
        const float M = mp[0], invL = mp[1];
        mq[qt][r] = invL > 0.f ? M - __log2f(invL) : INFINITY;
      }
  }
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  // one tile = 64 rows x D: 64*D*2/1024 copies of 1 KB, spread over the waves
  constexpr int kCopies = 64 * D * 2 / 1024;
  static_assert(kCopies % kVsWaves == 0, "every wave issues the same number of copies per tile");
  auto copy = [&](int tl, int buf) {
    for (int n = wv; n < kCopies; n += kVsWaves) {
      const int r = (1024 / (D * 2)) * n + lane / CPR, cpos = lane % CPR;
      const int c = D == 128 ? (cpos ^ (r & 15)) : (cpos ^ ((r >> 1) & 7));
      const int64_t grow = std::min((tb + tl) * 64 + r, N - 1);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(&Kt[buf][0]) + (uint32_t)n * 1024u);
      dma16(dst, kb + grow * D + 8 * c);
    }
  };
  // Pass 1 keeps two tiles in flight: its loop issues no other memory
  // operation, so waiting until one tile's copies (kCopies / kVsWaves per
  // wave) remain outstanding means tile tl has landed.  Pass 2 (no room for a
  // third tile in LDS) waits for its one copy in flight.
  constexpr int kCpw = kCopies / kVsWaves;
  if (nt > 0) copy(0, 0);
  if (!PASS2 && nt > 1) copy(1, 1);
  for (int tl = 0; tl < nt; ++tl) {
    const int buf = tl % NB;
    if (!PASS2 && tl + 1 < nt) wait_vmcnt<kCpw>();
    else wait_vmcnt<0>();
    __syncthreads();  // tile tl landed; the buffer refilled next and the P tiles are free
    if (tl + NB - 1 < nt) copy(tl + NB - 1, (tl + NB - 1) % NB);
    const int64_t s0 = (tb + tl) * 64;
    const bool last = s0 + 64 == N;
    if (active) {
      bf16x8 kr[NS];
      const int kr_row = 32 * kh + l32;
#pragma unroll
      for (int s4 = 0; s4 < NS; ++s4)
        kr[s4] = as_bf16x8(*reinterpret_cast<const u32x4*>(&Kt[buf][kr_row * D + 8 * vs_swz<D>(kr_row, 2 * s4 + hf)]));
      if constexpr (!PASS2) {
        // S^T[key][query]: lane = query 32qt + l32, rows = keys 32kh + 8(r/4) + 4hf + r%4
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          f32x16 acc = mfma32x32x16(kr[0], qv[qt][0], f32x16{});
#pragma unroll
          for (int s4 = 1; s4 < NS; ++s4) acc = mfma32x32x16(kr[s4], qv[qt][s4], acc);
          // only the last tile holds keys past a query (the queries are the last 64 positions)
          if (last) {
            const int qloc = 32 * qt + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * kh + 8 * (r / 4) + 4 * hf + (r % 4) > qloc) acc[r] = -INFINITY;
          }
          // the maximum of the raw scores, scaled once (sl2 > 0)
          float mx = acc[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[r]);
          mx = xor32_max(mx) * sl2;
          const float mnew = fmaxf(m[qt], mx);
          const float muse = mnew == -INFINITY ? 0.f : mnew;
          float ps = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) ps += fast_exp2(fmaf(acc[r], sl2, -muse));
          ps = xor32_add(ps);
          l[qt] = l[qt] * fast_exp2(m[qt] - muse) + ps;
          m[qt] = mnew;
        }
      } else {
        // S[query][key]: lane = key 32kh + l32, rows = queries 32qt + 8(r/4) + 4hf + r%4
        const int64_t key = s0 + 32 * kh + l32;
        float cs = 0.f;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          f32x16 acc = mfma32x32x16(qv[qt][0], kr[0], f32x16{});
#pragma unroll
          for (int s4 = 1; s4 < NS; ++s4) acc = mfma32x32x16(qv[qt][s4], kr[s4], acc);
          float pv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = 32 * qt + 8 * (r / 4) + 4 * hf + (r % 4);
            pv[r] = fast_exp2(fmaf(acc[r], sl2, -mq[qt][r]));
            if (last && 32 * kh + l32 > qi) pv[r] = 0.f;  // key past the query: last tile only
            cs += pv[r];
          }
          // P^T row of this key: four consecutive queries per 16-byte store
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<f32x4*>(&Pl[js][32 * kh + l32][32 * qt + 8 * r4 + 4 * hf]) =
                f32x4{pv[4 * r4], pv[4 * r4 + 1], pv[4 * r4 + 2], pv[4 * r4 + 3]};
        }
        cs = xor32_add(cs);
        if (hf == 0) av_s[js][tl * 64 + 32 * kh + l32] = cs;
      }
    }
    if constexpr (PASS2) {
      __syncthreads();  // every slot's P tile is in LDS
      // Diagonals d = query - key in [-63, 63].  The cyclic diagonal p
      // (query = (key + p) mod 64) holds d = p for keys < 64 - p and d = p - 64
      // for the rest: 64 elements, so every lane does the same work.  Slot
      // tid/128; p = 32 * (wave in slot) + lane%32; lane half hh sums keys
      // 32hh .. 32hh+31 (the halves read distinct banks), combined by one
      // exchange.
      const int jj = tid >> 7, pc = 32 * ((tid >> 6) & 1) + l32;
      if (rows[jj] >= 0) {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int e0 = 0; e0 < 32; e0 += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int e = 32 * hf + e0 + u;
            v[u] = Pl[jj][e][(e + pc) & 63];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (32 * hf + e0 + u < 64 - pc) sa += v[u];
            else sb += v[u];
          }
        }
        sa = xor32_add(sa);
        sb = xor32_add(sb);
        if (hf == 0) {
          dp_s[jj][tl][pc + 63] = sa;           // d = pc
          if (pc > 0) dp_s[jj][tl][pc - 1] = sb;  // d = pc - 64
        }
      }
    }
  }
  if constexpr (PASS2) {
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (rows[jj] < 0) continue;
      for (int i = tid; i < nt * 64; i += 64 * kVsWaves) a_v[(int64_t)rows[jj] * N + tb * 64 + i] = av_s[jj][i];
      for (int i = tid; i < nt * 128; i += 64 * kVsWaves)
        if ((i & 127) < 127) dpart[((int64_t)rows[jj] * ntile + tb) * 128 + i] = dp_s[jj][i >> 7][i & 127];
    }
  }
  if constexpr (!PASS2) {
    // merge the two key halves of each head slot, then one write per query
    if (active && hf == 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        st[js][kh][32 * qt + l32][0] = m[qt];
        st[js][kh][32 * qt + l32][1] = l[qt];
      }
    }
    __syncthreads();
    if (active && kh == 0 && hf == 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int qi = 32 * qt + l32;
        const float m0 = st[js][0][qi][0], l0 = st[js][0][qi][1], m1 = st[js][1][qi][0], l1 = st[js][1][qi][1];
        const float M = fmaxf(m0, m1);
        const float Mu = M == -INFINITY ? 0.f : M;
        float* sp = stats + (((int64_t)row * nchunk + ck) * kVsLast + qi) * 2;
        sp[0] = M;
        sp[1] = l0 * fast_exp2(m0 - Mu) + l1 * fast_exp2(m1 - Mu);
      }
    }
  }
}

// Merge of the per-chunk statistics: thread = (row, query); 8 chunks' loads in
// flight, chunks combined in order.
__global__ __launch_bounds__(64) void k_vs_stats_merge(const float* __restrict__ stats, int nchunk, float* __restrict__ ml) {
  const int bh = blockIdx.x, r = threadIdx.x;
  const float* sp0 = stats + ((int64_t)bh * nchunk * kVsLast + r) * 2;
  constexpr int U = 8;
  float M = -INFINITY;
  for (int c0 = 0; c0 < nchunk; c0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = c0 + u < nchunk ? sp0[(int64_t)(c0 + u) * kVsLast * 2] : -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, v[u]);
  }
  const float Mu = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  for (int c0 = 0; c0 < nchunk; c0 += U) {
    float mv[U], lv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = c0 + u < nchunk;
      mv[u] = in ? sp0[(int64_t)(c0 + u) * kVsLast * 2] : -INFINITY;
      lv[u] = in ? sp0[(int64_t)(c0 + u) * kVsLast * 2 + 1] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) L += lv[u] * fast_exp2(mv[u] - Mu);
  }
  ml[((int64_t)bh * kVsLast + r) * 2] = Mu;
  ml[((int64_t)bh * kVsLast + r) * 2 + 1] = L > 0.f ? 1.f / L : 0.f;
}

// a_s[o] = sum over the (at most two) tiles whose diagonals reach offset o
__global__ __launch_bounds__(256) void k_vs_slash(const float* __restrict__ dpart, int64_t N, int rows,
                                                  float* __restrict__ a_s, const float* __restrict__ a_v,
                                                  int32_t* __restrict__ err) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)rows * N) return;
  const int64_t bh = e / N, o = e % N;
  const int64_t ntile = (N + 63) / 64;
  const int64_t base = N - kVsLast - o;  // delta = o - (N - 64 - 64 tau) = 64 tau - base
  int64_t tlo = (base - 63 + 63) / 64;   // ceil((base-63)/64) for base-63 >= 0
  if (base - 63 < 0) tlo = -((63 - base) / 64);
  const int64_t thi = (base + 63) >= 0 ? (base + 63) / 64 : -1;
  float s = 0.f;
  for (int64_t tau = std::max<int64_t>(0, tlo); tau <= std::min(ntile - 1, thi); ++tau) {
    const int64_t delta = 64 * tau - base;
    if (delta >= -63 && delta <= 63) s += dpart[(bh * ntile + tau) * 128 + delta + 63];
  }
  a_s[e] = s;
  if (err != nullptr) flag_nonfinite(err, nonfinite(s) || nonfinite(a_v[e]));  // a_v has the same layout
}

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

hipError_t launch_indexer(const uint16_t* q, const uint16_t* k, const float* w, int T, int hi, int64_t nk,
                          int64_t pos0, float* out, int32_t* err, hipStream_t stream) {
  const int nchunk = (int)((nk + kIdxChunk - 1) / kIdxChunk);
  IdxCand flag{};
  flag.err = err;  // the dense scores only use the flag
  if (const hipError_t e = scan_indexer_inputs(q, k, w, T, hi, nk, err, stream); e != hipSuccess) return e;
  if (hi == 32) {
    constexpr int nq = kIdx2Waves * idx2_qpw<1>();
    const dim3 grid2((unsigned)(((T + nq - 1) / nq) * nchunk));
    hipLaunchKernelGGL((k_indexer2<1, false>), grid2, dim3(64 * kIdx2Waves), 0, stream, q, k, w, T, hi, nk, 1, kIdxChunk,
                       pos0, out, flag);
    return hipGetLastError();
  }
  if (hi == 64) {
    constexpr int nq = kIdx2Waves * idx2_qpw<2>();
    const dim3 grid2((unsigned)(((T + nq - 1) / nq) * nchunk));
    hipLaunchKernelGGL((k_indexer2<2, false>), grid2, dim3(64 * kIdx2Waves), 0, stream, q, k, w, T, hi, nk, 1, kIdxChunk,
                       pos0, out, flag);
    return hipGetLastError();
  }
  // the other multiples of 8 up to 64 heads: hi / 8 heads per wave
  const dim3 grid((unsigned)(((T + 31) / 32) * nchunk));
  const int hpw = hi / kIdxWaves;
#define SA_IDX_CASE(H_)                                                                                              \
  case H_:                                                                                                           \
    hipLaunchKernelGGL((k_indexer<H_>), grid, dim3(64 * kIdxWaves), 0, stream, q, k, w, T, hi, nk, pos0, out, err); \
    break;
  switch (hpw) {
    SA_IDX_CASE(1)
    SA_IDX_CASE(2)
    SA_IDX_CASE(3)
    SA_IDX_CASE(5)
    SA_IDX_CASE(6)
    SA_IDX_CASE(7)
    default: return hipErrorInvalidValue;
  }
#undef SA_IDX_CASE
  return hipGetLastError();
}

namespace {
struct IdxTopkLayout {
  int64_t ns, nseg, rs;
  int expect;
  size_t o_thr, o_segc, o_cand, bytes;
};
IdxTopkLayout idx_topk_layout(int T, int64_t nk, int64_t pos0, int k) {
  IdxTopkLayout L;
  L.ns = (nk + kIdxStride - 1) / kIdxStride;
  L.expect = kIdxExpect;
  const int64_t nmax = std::min(nk, pos0 + T);
  L.nseg = (nmax + kIdxChunk - 1) / kIdxChunk;
  L.rs = (2 * (int64_t)L.expect + 128 * L.nseg + 63) / 64 * 64;
  (void)k;  // the layout does not depend on k (at most 2048)
  L.o_thr = nmax > kIdxSelCap ? a256((size_t)T * L.ns * 4) : 0;  // sampled scores only for long rows
  L.o_segc = L.o_thr + a256((size_t)T * 4);
  L.o_cand = L.o_segc + a256((size_t)(T * L.nseg) * 4);
  L.bytes = L.o_cand + a256((size_t)(T * L.rs) * 8);
  return L;
}
}  // namespace

size_t indexer_topk_workspace_bytes(int T, int64_t nk, int64_t pos0, int k) {
  return idx_topk_layout(T, nk, pos0, k).bytes;
}

hipError_t launch_indexer_topk(const uint16_t* q, const uint16_t* k, const float* w, int T, int hi, int64_t nk,
                               int64_t pos0, int kk, int kmax, int32_t* idx, int32_t* cnt, int32_t* err, void* ws,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (hi != 32 && hi != 64) return hipErrorInvalidValue;
  if (const hipError_t e = scan_indexer_inputs(q, k, w, T, hi, nk, err, stream); e != hipSuccess) return e;
  const IdxTopkLayout L = idx_topk_layout(T, nk, pos0, kk);
  char* base = static_cast<char*>(ws);
  float* smp = reinterpret_cast<float*>(base);
  IdxCand cd;
  float* thr = reinterpret_cast<float*>(base + L.o_thr);
  cd.thr = thr;
  cd.segc = reinterpret_cast<int32_t*>(base + L.o_segc);
  cd.cand = reinterpret_cast<int2*>(base + L.o_cand);
  cd.err = err;
  cd.rs = L.rs;
  cd.nseg = (int)L.nseg;
  cd.expect = L.expect;
  const int nq = kIdx2Waves * (hi == 32 ? idx2_qpw<1>() : idx2_qpw<2>());
  const unsigned nqt = (unsigned)((T + nq - 1) / nq);
  const dim3 g_smp(nqt * (unsigned)((L.ns + kIdxSampleChunk - 1) / kIdxSampleChunk));
  const dim3 g_full(nqt * (unsigned)((nk + kIdxChunk - 1) / kIdxChunk));
  const dim3 blk(64 * kIdx2Waves);
  if (std::min(nk, pos0 + T) > kIdxSelCap) {  // some row is long enough to need the sampled threshold
    if (hi == 32)
      hipLaunchKernelGGL((k_indexer2<1, false>), g_smp, blk, 0, stream, q, k, w, T, hi, L.ns, kIdxStride,
                         kIdxSampleChunk, pos0, smp, IdxCand{});
    else
      hipLaunchKernelGGL((k_indexer2<2, false>), g_smp, blk, 0, stream, q, k, w, T, hi, L.ns, kIdxStride,
                         kIdxSampleChunk, pos0, smp, IdxCand{});
  }
  hipLaunchKernelGGL(k_idx_thresh, dim3((unsigned)T), dim3(256), 0, stream, smp, L.ns, nk, pos0, thr, err);
  if (hi == 32)
    hipLaunchKernelGGL((k_indexer2<1, true>), g_full, blk, 0, stream, q, k, w, T, hi, nk, 1, kIdxChunk, pos0,
                       nullptr, cd);
  else
    hipLaunchKernelGGL((k_indexer2<2, true>), g_full, blk, 0, stream, q, k, w, T, hi, nk, 1, kIdxChunk, pos0,
                       nullptr, cd);
  hipLaunchKernelGGL(k_idx_select, dim3((unsigned)T), dim3(kIdxSelNT), 0, stream, cd, nk, pos0, kIdxChunk, kk, kmax,
                     idx, cnt);
  return hipGetLastError();
}

size_t vs_workspace_bytes(int64_t rows, int64_t seq) {
  const int64_t ntile = (seq + 63) / 64;
  const int64_t nchunk = (ntile + kVsTilesPerWg - 1) / kVsTilesPerWg;
  return a256((size_t)(rows * nchunk * kVsLast * 2) * 4) + a256((size_t)(rows * kVsLast * 2) * 4) +
         a256((size_t)(rows * ntile * 128) * 4);
}

hipError_t launch_vs_estimate(const uint16_t* q, const uint16_t* k, int batch, int hq, int hkv,
                              const HeadList& hl, int64_t seq, int head_dim, int last_q, float scale, float* a_v,
                              float* a_s, int32_t* err, void* ws, hipStream_t stream) {
  if (last_q != kVsLast) return hipErrorInvalidValue;
  const int rows = batch * (hl.n > 0 ? hl.n : hq);
  const int64_t ntile = (seq + 63) / 64;
  const int nchunk = (int)((ntile + kVsTilesPerWg - 1) / kVsTilesPerWg);
  char* p = static_cast<char*>(ws);
  float* stats = reinterpret_cast<float*>(p);
  p += a256((size_t)((int64_t)rows * nchunk * kVsLast * 2) * 4);
  float* ml = reinterpret_cast<float*>(p);
  p += a256((size_t)((int64_t)rows * kVsLast * 2) * 4);
  float* dpart = reinterpret_cast<float*>(p);
  const float sl2 = scale * kLog2e;
  const int grp = hq / hkv, nhs = (grp + 3) / 4;
  const dim3 grid((unsigned)((int64_t)batch * hkv * nhs * nchunk)), blk(64 * kVsWaves);
  if (head_dim == 128) {
    hipLaunchKernelGGL((k_vs_pass<128, false>), grid, blk, 0, stream, q, k, hq, hkv, hl, seq, sl2, nchunk, nhs,
                       nullptr, stats, nullptr, nullptr);
    hipLaunchKernelGGL(k_vs_stats_merge, dim3(rows), dim3(64), 0, stream, stats, nchunk, ml);
    hipLaunchKernelGGL((k_vs_pass<128, true>), grid, blk, 0, stream, q, k, hq, hkv, hl, seq, sl2, nchunk, nhs, ml,
                       nullptr, a_v, dpart);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL((k_vs_pass<64, false>), grid, blk, 0, stream, q, k, hq, hkv, hl, seq, sl2, nchunk, nhs,
                       nullptr, stats, nullptr, nullptr);
    hipLaunchKernelGGL(k_vs_stats_merge, dim3(rows), dim3(64), 0, stream, stats, nchunk, ml);
    hipLaunchKernelGGL((k_vs_pass<64, true>), grid, blk, 0, stream, q, k, hq, hkv, hl, seq, sl2, nchunk, nhs, ml,
                       nullptr, a_v, dpart);
  } else {
    return hipErrorInvalidValue;
  }
  const int64_t n = (int64_t)rows * seq;
  hipLaunchKernelGGL(k_vs_slash, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dpart, seq, rows, a_s, a_v,
                     err);
  return hipGetLastError();
}

}  // namespace sa
