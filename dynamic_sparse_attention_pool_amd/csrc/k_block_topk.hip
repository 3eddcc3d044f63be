// Block-sparse estimate and selection in one pass: pooled block scores reduced
// to each query-block row's kept set without writing the score matrix.
//
// "MInference 1.0" article, §方法介紹: block indices come from the product of
// mean-pooled Q and K; the top blocks of each row are kept, together with the
// always-attended sink and local blocks ("稀疏注意力机制解析" explainer, §1.2).
// Same result as the pooled scores followed by the per-row top-k: the score of
// a causal pair is Qbar_i . Kbar_j * scale, the order is higher score first and
// lower index on ties, forced blocks are kept and not counted in the budget.
//
// One workgroup (8 waves) takes 16 consecutive query-block rows of one head:
//   scores — v_mfma_f32_16x16x4_f32 with the 16 rows on the A side and 16
//     candidate blocks per tile on the B side.  Dimension 16q + 4c + e goes to
//     k-slot c of step 4q + e, so every lane loads its operands with 16-byte
//     loads and the 4 k-slot lanes of one candidate read 64 adjacent bytes
//     (the dot product does not depend on how dimensions map to steps).  The
//     operands of the next two tiles are in flight while a tile's steps run
//     on two accumulators.  Tile t goes to wave t % 8, so
//     the causal triangle is shared evenly; each lane keeps its 16 tiles x 4
//     rows of scores in registers as order-preserving keys (0 = not in the
//     pool: forced, not causal or past the last block).
//   threshold — per row, the k-th largest pool key T by an MSB-first radix
//     select: 4 passes of 8-bit digits, each building the rows' 256-bin
//     histograms of the keys that match the digits chosen so far (LDS
//     atomics), then 32 threads per row find the digit where the count from
//     the top reaches the remaining k.
//   emission — per (row, tile) counts of kept-for-sure entries (forced or
//     above T) and of ties (== T) go to LDS, an exclusive scan over the tiles
//     in index order gives every entry its output position, and the first
//     `k - #above` ties in index order are kept.
#include "common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kTkRows = 16;
constexpr int kTkWaves = 8;
constexpr int kTkSlots = 16;                  // tiles per wave
constexpr int kTkTiles = kTkWaves * kTkSlots;  // 128 tiles of 16 = 2048 candidate blocks

__device__ __forceinline__ uint32_t group16_mask(uint64_t ballot, int grp) {
  return (uint32_t)(ballot >> (16 * grp)) & 0xffffu;
}

// Operands of one lane: the 16-byte chunks c, c+4, c+8, ... of a row (c = the
// lane's k-slot); chunk 4q + c feeds steps 4q .. 4q+3.
template <int D>
__device__ __forceinline__ void load_slot(float* dst, const float* src) {
  constexpr int ST = D / 4;
#pragma unroll
  for (int q = 0; q < ST / 4; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + 16 * q);
    dst[4 * q] = v[0];
    dst[4 * q + 1] = v[1];
    dst[4 * q + 2] = v[2];
    dst[4 * q + 3] = v[3];
  }
}

template <int D>
__global__ __launch_bounds__(64 * kTkWaves) void k_block_topk(BlockTopkParams p) {
  constexpr int ST = D / 4;  // MFMA steps per tile: each k-slot covers D/4 contiguous dimensions
  __shared__ uint32_t s_hist[kTkRows][256];
  __shared__ uint32_t s_digit[kTkRows][2];
  __shared__ int32_t s_need[kTkRows];
  __shared__ uint32_t s_fg[kTkRows][kTkTiles];
  __shared__ uint32_t s_tie[kTkRows][kTkTiles];
  __shared__ uint32_t s_nan;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const int npanel = (p.nb + kTkRows - 1) / kTkRows;
  const int64_t bh = blockIdx.x / npanel;
  const int i0 = (npanel - 1 - (int)(blockIdx.x % npanel)) * kTkRows;  // long rows first
  int b, h;
  listed_row(bh, p.hq, p.hl, b, h);
  const int g = h * p.hkv / p.hq;
  const float* qbar = p.pq + bh * p.nb * D;
  const float* kbar = p.pk + ((int64_t)b * p.hkv + g) * p.nb * D;
  const int ncand = min(p.nb, i0 + kTkRows);
  const int ntile = (ncand + 15) / 16;
  const int mv = (ntile - w + kTkWaves - 1) / kTkWaves;  // tiles of this wave (wave-uniform)
  if (tid == 0) s_nan = 0u;
  for (int e = tid; e < kTkRows * kTkTiles; e += 64 * kTkWaves) {
    (&s_fg[0][0])[e] = 0u;
    (&s_tie[0][0])[e] = 0u;
  }

  // rows of this lane's group and their pool ranges [pb, pe) and budgets
  int pb[4], pe[4], kr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * grp + r;
    const int n = i + 1;
    pb[r] = min(p.n_sink, n);
    pe[r] = max(pb[r], n - p.n_local);
    const int npool = pe[r] - pb[r];
    int64_t kk = p.rden > 0 ? ((int64_t)p.rnum * n + p.rden - 1) / p.rden : (int64_t)p.k;
    kk = max((int64_t)0, min(kk, (int64_t)npool));
    kr[r] = i < p.nb ? (int)kk : 0;
  }

  // A operand: row i0 + c16, dimensions [grp*ST, grp*ST + ST)
  // Rows and candidates past the last block read block nb-1 (in bounds); their
  // keys are never used.  Loads are unconditional so that no branch makes the
  // compiler wait for the tiles in flight.
  float qa[ST];
  load_slot<D>(qa, qbar + (int64_t)min(i0 + c16, p.nb - 1) * D + 4 * grp);
  const int jlast = min(p.nb, 16 * (kTkWaves * max(mv - 1, 0) + w) + 16) - 1;  // last candidate of the wave

  // ---- scores -> keys in registers; tiles m+1 and m+2 load during tile m
  uint32_t key[kTkSlots][4];
  bool nan_seen = false;
  float kb[3][ST];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int j = min(16 * (kTkWaves * m + w) + c16, max(jlast, 0));
    load_slot<D>(kb[m], kbar + (int64_t)j * D + 4 * grp);
  }
#pragma unroll
  for (int m = 0; m < kTkSlots; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) key[m][r] = 0u;
    if (m + 2 < kTkSlots) {
      const int jn = min(16 * (kTkWaves * (m + 2) + w) + c16, max(jlast, 0));
      load_slot<D>(kb[(m + 2) % 3], kbar + (int64_t)jn * D + 4 * grp);
    }
    if (m < mv) {
      const int j = 16 * (kTkWaves * m + w) + c16;
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < ST; s += 2) {
        a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[s], kb[m % 3][s], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[s + 1], kb[m % 3][s + 1], a1, 0, 0, 0);
      }
      const f32x4 acc = a0 + a1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // D[4*grp + r][c16]: row i0 + 4*grp + r, candidate j
        const int i = i0 + 4 * grp + r;
        const float sc = acc[r] * p.scale;
        const bool causal = i < p.nb && j <= i;
        nan_seen |= causal && is_nan(sc);
        key[m][r] = (causal && j >= pb[r] && j < pe[r]) ? order_key(sc) : 0u;
      }
    }
  }
  __syncthreads();
  if (nan_seen) atomicOr(&s_nan, 1u);

  // ---- threshold: the k-th largest pool key of each row (radix select, 8-bit digits)
  constexpr int TPR = 64 * kTkWaves / kTkRows;  // threads per row in the digit search (32)
  uint32_t T[4] = {0u, 0u, 0u, 0u};
  int need[4] = {kr[0], kr[1], kr[2], kr[3]};
  if (w == 0 && c16 == 0)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_need[4 * grp + r] = need[r];
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    const uint32_t hmask = shift == 24 ? 0u : ~((1u << (shift + 8)) - 1u);  // digits already chosen
    for (int e = tid; e < kTkRows * 256; e += 64 * kTkWaves) (&s_hist[0][0])[e] = 0u;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kTkSlots; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t k = key[m][r];
        if (m < mv && k != 0u && (k & hmask) == (T[r] & hmask))
          atomicAdd(&s_hist[4 * grp + r][(k >> shift) & 255u], 1u);
      }
    __syncthreads();
    {
      const int row = tid / TPR, seg = tid % TPR;  // seg owns bins [8*seg, 8*seg + 8)
      const int rneed = s_need[row];
      uint32_t loc = 0u;
#pragma unroll
      for (int x = 0; x < 8; ++x) loc += s_hist[row][8 * seg + x];
      // count of the bins above this segment: inclusive scan from the top segment down
      uint32_t incl = loc;
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) {
        const uint32_t o = __shfl_down(incl, off, TPR);
        if (seg + off < TPR) incl += o;
      }
      const uint32_t above = incl - loc;
      if (rneed == 0) {
        if (seg == TPR - 1) {
          s_digit[row][0] = 255u;
          s_digit[row][1] = 0u;
        }
      } else if (above < (uint32_t)rneed && (uint32_t)rneed <= incl) {
        uint32_t acc = above;
        for (int d = 8 * seg + 7; d >= 8 * seg; --d) {
          const uint32_t hcount = s_hist[row][d];
          if (acc + hcount >= (uint32_t)rneed) {
            s_digit[row][0] = (uint32_t)d;
            s_digit[row][1] = acc;
            break;
          }
          acc += hcount;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      T[r] |= s_digit[4 * grp + r][0] << shift;
      need[r] -= (int)s_digit[4 * grp + r][1];
    }
    if (w == 0 && c16 == 0)  // read again only after the next two barriers
#pragma unroll
      for (int r = 0; r < 4; ++r) s_need[4 * grp + r] = need[r];
  }

  // ---- per (row, tile): entries kept for sure (forced or above T) and ties
  // (tiles past the wave's last stay at the zeros written at the start)
#pragma unroll
  for (int m = 0; m < kTkSlots; ++m) {
    if (m < mv) {  // wave-uniform
      const int t = kTkWaves * m + w;
      const int j = 16 * t + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * grp + r;
        const bool causal = m < mv && i < p.nb && j <= i;
        const bool forced = causal && (j < pb[r] || j >= pe[r]);
        const bool fg = forced || key[m][r] > T[r];
        const bool tie = !fg && key[m][r] != 0u && key[m][r] == T[r];
        const uint32_t mf = group16_mask(__ballot(fg), grp), mt = group16_mask(__ballot(tie), grp);
        if (c16 == 0) {
          s_fg[4 * grp + r][t] = (uint32_t)__popc(mf);
          s_tie[4 * grp + r][t] = (uint32_t)__popc(mt);
        }
      }
    }
  }
  __syncthreads();
  // exclusive scan over the 128 tiles of each row: 32 threads per row, 4 tiles each
  {
    constexpr int TPR = 64 * kTkWaves / kTkRows, TPS = kTkTiles / TPR;
    const int row = tid / TPR, seg = tid % TPR;
    uint32_t f8 = 0u, t8 = 0u;
#pragma unroll
    for (int x = 0; x < TPS; ++x) {
      f8 += s_fg[row][TPS * seg + x];
      t8 += s_tie[row][TPS * seg + x];
    }
    uint32_t fi = f8, ti = t8;  // inclusive scan over the segments of the row (consecutive lanes)
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) {
      const uint32_t fo = __shfl_up(fi, off), to = __shfl_up(ti, off);
      if (seg >= off) {
        fi += fo;
        ti += to;
      }
    }
    uint32_t fr = fi - f8, tr = ti - t8;
#pragma unroll
    for (int x = 0; x < TPS; ++x) {
      const uint32_t a = s_fg[row][TPS * seg + x], e = s_tie[row][TPS * seg + x];
      s_fg[row][TPS * seg + x] = fr;
      s_tie[row][TPS * seg + x] = tr;
      fr += a;
      tr += e;
    }
  }
  __syncthreads();

  // ---- emission in index order
  const uint32_t below = (1u << c16) - 1u;
#pragma unroll
  for (int m = 0; m < kTkSlots; ++m) {
    if (m < mv) {  // wave-uniform
      const int t = kTkWaves * m + w;
      const int j = 16 * t + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * grp + r;
        const int i = i0 + row;
        const bool causal = m < mv && i < p.nb && j <= i;
        const bool forced = causal && (j < pb[r] || j >= pe[r]);
        const bool fg = forced || key[m][r] > T[r];
        const bool tie = !fg && key[m][r] != 0u && key[m][r] == T[r];
        const uint32_t mf = group16_mask(__ballot(fg), grp), mt = group16_mask(__ballot(tie), grp);
        if (fg || tie) {
          const int fb = (int)s_fg[row][t] + __popc(mf & below);
          const int tb = (int)s_tie[row][t] + __popc(mt & below);
          int32_t* out = p.idx + (bh * p.nb + i) * p.kmax;
          if (fg) out[fb + min(tb, need[r])] = j;
          else if (tb < need[r]) out[fb + tb] = j;
        }
      }
    }
  }
  // counts and -1 padding
  for (int e = tid; e < kTkRows * p.kmax; e += 64 * kTkWaves) {
    const int row = e / p.kmax, pos = e % p.kmax;
    const int i = i0 + row;
    if (i >= p.nb) continue;
    const int n = i + 1;
    const int pbr = min(p.n_sink, n), per = max(pbr, n - p.n_local);
    int64_t kk = p.rden > 0 ? ((int64_t)p.rnum * n + p.rden - 1) / p.rden : (int64_t)p.k;
    kk = max((int64_t)0, min(kk, (int64_t)(per - pbr)));
    const int total = pbr + (n - per) + (int)kk;
    if (pos >= total) p.idx[(bh * p.nb + i) * p.kmax + pos] = -1;
    if (pos == 0) p.cnt[bh * p.nb + i] = total;
  }
  if (tid == 0 && s_nan && p.err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(p.err), 1u);
}

}  // namespace

hipError_t launch_block_topk(const BlockTopkParams& p, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * (p.hl.n > 0 ? p.hl.n : p.hq);
  const int64_t n = rows * ((p.nb + kTkRows - 1) / kTkRows);
  if (n == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL((k_block_topk<128>), dim3((unsigned)n), dim3(64 * kTkWaves), 0, stream, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_block_topk<64>), dim3((unsigned)n), dim3(64 * kTkWaves), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
