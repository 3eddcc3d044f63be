// Block-sparse / vertical-slash attention forward for gfx950.
//
// "MInference 1.0" article, §方法介紹: exact attention runs only over the
// estimated blocks with a FlashAttention-style kernel; §延遲和內核中的稀疏模式,
// Fig. 4: the vertical-slash kernel covers slash lines with 64x64 tiles and
// vertical lines with 1x64 column pieces.  Both reduce to one loop: for a
// 64-row query block, visit a list of 64-key tiles (contiguous ranges or
// gathered columns), and fold each into an online softmax.
//
// bf16 kernel — one workgroup (2 waves) per (batch, head, query block); each
// wave owns 32 query rows.  Per tile:
//   K and V rows are copied straight from memory into LDS by the direct
//   global->LDS path (global_load_lds_dwordx4), row-major with the 16-byte
//   chunks of each row XOR-swizzled by a key of the row index, so no VGPR
//   staging and no bank conflicts;
//   S^T[key][query] = K_tile . Q^T          (v_mfma_f32_32x32x16_bf16, K from LDS,
//                                            Q^T resident in VGPRs)
//   online softmax along keys: every lane holds one query column, so the row
//   statistics need a single exchange with lane^32 (a register lane swap)
//   O^T[d][query] += V^T . P^T               (V^T read with ds_read_b64_tr_b16, which
//                                            transposes 4-key x 16-dim blocks on the
//                                            way out of LDS; P^T comes straight from
//                                            the S^T accumulators, no shuffles)
// The probabilities of each 8-key step are made just before that step's P.V
// products, so the exps overlap the matrix core; in block mode the first half
// of them is made with the current reference maximum before the tile's own
// maximum is known.  K(t+1) is fetched while the softmax and P.V of tile t
// run, V(t+1) while the next S^T runs: one LDS buffer each (40 KB per
// workgroup, four workgroups per CU), four barriers per tile.  Every kept
// (head, query block, key block) brings its own 32 KB of K and V through L2;
// with all of them L2 hits the loop still takes most of the time, its VALU
// softmax and its products overlapping only in part.
#include <climits>

#include "common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kBlk = 64;
constexpr int kThreads = 128;
constexpr int kMetaMax = 2048;        // staged block list, or 64 intervals + up to 1920 columns
constexpr int kMaxCols = kMetaMax - 128;
constexpr float kSlack = 8.f;         // lazy-rescale threshold, log2 units

// Tile source: either a contiguous key range or a gathered list of columns.
struct TileRef {
  int base;      // first key (contiguous) or offset into the column list (gathered)
  int len;       // valid keys, 1..64
  int gathered;  // 0 / 1
  int diag;      // tile may hold keys beyond some query row of the block
};

template <int MODE>
struct TileIter {
  // block mode; `pre` holds entry t, read one call ahead so the LDS latency
  // of the next index is hidden behind a whole tile
  const int32_t* bidx = nullptr;
  int cnt = 0, t = 0, iblk = 0, pre = -1;
  // vertical-slash mode
  const int32_t* iv = nullptr;
  const int32_t* col = nullptr;  // ascending column list (optional: without it every column tile is masked)
  int n_iv = 0, cur_iv = 0, cur_off = 0;
  int n_col = 0, col_off = 0;
  int lim = 0;          // keys at or beyond min(seq, end of the query block) are never loaded
  int bad_cols = 0;     // some column lies outside [0, seq): mask every gathered tile

  // block mode: read the first entry once bidx and cnt are set (and the list,
  // when staged in LDS, is visible to the whole workgroup)
  __device__ void start_blocks() { pre = cnt > 0 ? bidx[0] : -1; }

  __device__ bool next(TileRef& r) {
    if (MODE == 0) {
      int j = -1;
      while (t < cnt && (j < 0 || j > iblk)) {  // entries outside 0..i are skipped
        j = pre;
        ++t;
        pre = t < cnt ? bidx[t] : -1;
      }
      if (j < 0 || j > iblk) return false;
      r.base = j * kBlk;
      r.len = kBlk;
      r.gathered = 0;
      r.diag = (j == iblk);
      return true;
    }
    while (cur_iv < n_iv) {
      // an interval is clipped to [0, lim); an empty one is skipped
      const int s = max(iv[2 * cur_iv], 0), e = min(iv[2 * cur_iv + 1], lim);
      if (s + cur_off >= e) {
        ++cur_iv;
        cur_off = 0;
        continue;
      }
      r.base = s + cur_off;
      r.len = min(kBlk, e - r.base);
      r.gathered = 0;
      // masking only for a short tile or one reaching past the block's first query row
      r.diag = (r.len < kBlk) || (r.base + r.len - 1 > iblk * kBlk);
      cur_off += kBlk;
      return true;
    }
    if (col_off < n_col) {
      r.base = col_off;
      r.len = min(kBlk, n_col - col_off);
      r.gathered = 1;
      r.diag = (r.len < kBlk) || col == nullptr || bad_cols || (col[r.base + r.len - 1] > iblk * kBlk);
      col_off += kBlk;
      return true;
    }
    return false;
  }
};

// A listed column outside [0, seq) is never loaded: its copy reads row 0 and
// the key is masked.
__device__ __forceinline__ bool col_ok(int c, int64_t seq) { return c >= 0 && c < seq; }

__device__ __forceinline__ int tile_row(const TileRef& r, const int32_t* cols, int slot, int64_t seq) {
  const int s = min(slot, r.len - 1);
  if (!r.gathered) return r.base + s;
  const int c = cols[r.base + s];
  return col_ok(c, seq) ? c : 0;
}

// XOR key of row r: chunk c of row r sits at position c ^ key(r).  For d = 128
// the key is 4*(r%4) + (r/4)%4: sixteen consecutive rows get distinct keys (a
// 16-lane K read of one chunk hits 16 different bank groups) and the 4 rows x
// 4 chunks read by a half-wave of transposing V reads land on 16 different
// positions.  For d = 64 the key is r % 8.
template <int D>
__device__ __forceinline__ int swz_key(int row) {
  if (D == 128) return swz_key128(row);
  return row % (D / 8);
}

// One 64-row tile (K or V) -> LDS, row-major, chunk c of row r at position
// c ^ key(r).  Each wave issues NI copies of 1 KB at device scope.  A
// contiguous tile's first row goes into the 64-bit scalar base, so the lane
// offsets stay below 16 KB whatever the sequence length; a gathered tile
// gives every lane its own 64-bit address.
template <int D>
__device__ __forceinline__ void dma_tile(uint16_t* lds, const uint16_t* gbase, const TileRef& r,
                                         const int32_t* cols, int64_t seq, int w, int lane) {
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;       // rows per 1 KB copy
  constexpr int NI = kBlk / RPI / 2;  // copies per wave
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)(w * NI) * 1024u);
  if (!r.gathered) {
    const uint16_t* tb = gbase + (int64_t)__builtin_amdgcn_readfirstlane(r.base) * D;
    const int last = r.len - 1;
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int row = (w * NI + n) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz_key<D>(row);
      const uint32_t off = (uint32_t)min(row, last) * (uint32_t)(D * 2) + (uint32_t)(16 * c);
      dma16_sb_dev(base + (uint32_t)n * 1024u, tb, off);
    }
    return;
  }
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int row = (w * NI + n) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz_key<D>(row);
    dma16_dev(base + (uint32_t)n * 1024u, gbase + (int64_t)tile_row(r, cols, row, seq) * D + 8 * c);
  }
}

// Workgroup -> (head in group, query-block rank, batch x KV head).
// order 0: each XCD takes one contiguous range of items (a KV head per XCD
//          when batch x KV heads == 8).
// order 1: every XCD works on the same KV head at the same time, so the K/V
//          being read stays in the 256 MB Infinity Cache even when all heads'
//          K/V do not fit; each XCD takes runs of 4 consecutive query blocks
//          (neighbouring rows share their local blocks in that XCD's L2, and
//          all XCDs stay on nearby query blocks; runs of 2, 8, 16 and 32
//          measured slower or equal).  Needs nqb % 64 == 0 and the item count
//          a multiple of 8.
__device__ __forceinline__ void item_of(int bid, int n_items, int grp, int nqb, int order, int& hh, int& ii,
                                        int& bg) {
  if (order == 1) {
    const int x = bid % kXcds, slot = bid / kXcds;
    const int per_bg = (nqb / kXcds) * grp;  // items of one KV head on one XCD
    bg = slot / per_bg;
    const int rem = slot % per_bg;
    hh = rem % grp;
    const int r4 = (rem / grp) % 4;
    const int cidx = rem / (4 * grp);
    ii = (cidx * kXcds + x) * 4 + r4;
    return;
  }
  int rest = xcd_remap(bid, n_items);
  hh = rest % grp;
  rest /= grp;
  ii = rest % nqb;
  bg = rest / nqb;
}

// Workgroup -> batch b, query head h, query block iblk and the row of the index
// tables.  With a head list the launch's items are (b, listed head j), each its
// own group, and the tables are indexed compactly by b*n + j.
struct Item {
  int b, h, iblk;
  int64_t trow;
};

__device__ __forceinline__ Item item_at(const FwdParams& p, int bid, int n_items, int order) {
  const int grp = p.heads_q / p.heads_kv;
  int hh, ii, bg;
  Item it;
  if (p.hl.n > 0) {
    item_of(bid, n_items, 1, p.nqb, order, hh, ii, bg);
    it.b = bg / p.hl.n;
    it.h = p.hl.h[bg % p.hl.n];
  } else {
    item_of(bid, n_items, grp, p.nqb, order, hh, ii, bg);
    it.b = bg / p.heads_kv;
    it.h = (bg % p.heads_kv) * grp + hh;
  }
  it.iblk = p.nqb - 1 - ii;  // long rows first
  const int64_t r = p.hl.n > 0 ? (int64_t)bg : (int64_t)it.b * p.heads_q + it.h;
  it.trow = r * p.nqb + it.iblk;
  return it;
}

// A-shape rows need no table: blocks 0 .. n_sink-1 and the n_local blocks
// ending at the diagonal, ascending and each once.  Returns the count.
__device__ __forceinline__ int ashape_list(int32_t* dst, int iblk, int n_sink, int n_local, int tid, int nt) {
  const int se = min(n_sink, iblk + 1);
  const int lb = max(se, iblk - n_local + 1);
  const int cnt = se + (iblk + 1 - lb);
  for (int e = tid; e < cnt; e += nt) dst[e] = e < se ? e : lb + (e - se);
  return cnt;
}

// Element offset of 16-byte chunk `chunk` of row `row` in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * D + 8 * (chunk ^ swz_key<D>(row));
}

template <int D, int MODE, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void k_fwd_bf16(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t Kl[kBlk * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vl[kBlk * D];
  __shared__ int32_t meta[kMetaMax];  // with K and V: 40 KB, four workgroups per CU
  constexpr int NDMA = D / 16;  // direct-to-LDS copies per wave per tile (K or V)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, l32 = lane & 31;
  const Item item = item_at(p, blockIdx.x, gridDim.x, p.order);
  const int b = item.b, h = item.h, iblk = item.iblk;
  const int g = h / (p.heads_q / p.heads_kv);
  const int64_t N = p.seq;
  const int64_t row_id = item.trow;

  const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + (((int64_t)b * p.heads_q + h) * N + (int64_t)iblk * kBlk) * D;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.k) + ((int64_t)b * p.heads_kv + g) * N * D;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(p.v) + ((int64_t)b * p.heads_kv + g) * N * D;

  // ---- stage this row's tile list in LDS (no vector-memory reads inside the pipeline).
  //      Counts are clipped to the table capacities; intervals are clipped to
  //      the keys the block can see when they are read, and a column outside
  //      [0, seq) is loaded as row 0 and masked.
  TileIter<MODE> it;
  const int32_t* cols = nullptr;
  int bad_col = 0;
  if (MODE == 0) {
    int cnt;
    if (p.ashape) {
      cnt = ashape_list(meta, iblk, p.n_sink, p.n_local, tid, kThreads);
    } else {
      cnt = max(0, min(p.block_cnt[row_id], min(p.kmax, 2048)));
      const int32_t* src = p.block_idx + row_id * p.kmax;
      for (int e = tid; e < cnt; e += kThreads) meta[e] = src[e];
    }
    it.bidx = meta;
    it.cnt = cnt;
    it.iblk = iblk;
  } else {
    const int niv = max(0, min(p.iv_cnt[row_id], min(p.max_iv, 64)));
    const int ncol = max(0, min(p.col_cnt[row_id], min(p.max_col, kMaxCols)));
    const int32_t* isrc = p.iv + row_id * p.max_iv * 2;
    const int32_t* csrc = p.col + row_id * p.max_col;
    for (int e = tid; e < 2 * niv; e += kThreads) meta[e] = isrc[e];
    for (int e = tid; e < ncol; e += kThreads) {
      const int c = csrc[e];
      bad_col |= !col_ok(c, N);
      meta[128 + e] = c;
    }
    it.iv = meta;
    it.n_iv = niv;
    it.n_col = ncol;
    it.iblk = iblk;
    it.lim = (int)min(N, (int64_t)iblk * kBlk + kBlk);
    cols = meta + 128;
    it.col = cols;
  }

  // Q^T operand: lane holds query row 32w+l32, dims 16s+8hf .. +7 of step s
  bf16x8 qv[D / 16];
  {
    const uint16_t* qr = qb + (int64_t)(32 * w + l32) * D + 8 * hf;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qv[s] = as_bf16x8(ldg16(qr + 16 * s));
  }
  const int qpos = iblk * kBlk + 32 * w + l32;  // absolute query row of this lane
  const float sl2 = p.scale * kLog2e;
  drain_vmem();  // Q^T resident: from here on the only vector-memory ops are the tile copies
  if (MODE == 0) {
    __syncthreads();
    it.start_blocks();
  } else {
    // the row's bad-column flag passes through the K tile buffer, which no copy
    // has touched yet
    int* flag = reinterpret_cast<int*>(Kl);
    const int wbad = __any(bad_col);
    if (lane == 0) flag[w] = wbad;
    __syncthreads();
    it.bad_cols = flag[0] | flag[1];
    __syncthreads();  // both waves read the flags before the first copy lands
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  TileRef cur, nxt;
  bool have = it.next(cur);
  if (have) {
    dma_tile<D>(Kl, kb, cur, cols, N, w, lane);
    dma_tile<D>(Vl, vb, cur, cols, N, w, lane);
  }
  while (have) {
    // ---- K(t) in LDS
    wait_vmcnt<NDMA>();
    __builtin_amdgcn_s_barrier();
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
    {
      // keys 0..31 first, then 32..63 (operands of step st+1 read while step st
      // runs): the first half's scores are ready while the second half is
      // still on the matrix core
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x16& acc = half ? s1 : s0;
        bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&Kl[swz<D>(32 * half + l32, hf)]));
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          bf16x8 n = a;
          if (st + 1 < D / 16) n = as_bf16x8(*reinterpret_cast<const u32x4*>(&Kl[swz<D>(32 * half + l32, 2 * (st + 1) + hf)]));
          acc = mfma32x32x16(a, qv[st], acc);
          a = n;
        }
      }
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();  // both waves are done with K(t)
    const bool more = it.next(nxt);
    if (more) dma_tile<D>(Kl, kb, nxt, cols, N, w, lane);

    // ---- online softmax (log2 domain); element r of M tile mt is key slot
    //      32*mt + 8*(r/4) + 4*hf + r%4
    float x[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = s0[r];
      x[16 + r] = s1[r];
    }
    if (cur.diag) {
      if (MODE == 0) {
        const int lim = 32 * w + l32;  // slot index of this lane's own row
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          const int slot = 32 * (r / 16) + 8 * ((r % 16) / 4) + 4 * hf + (r % 4);
          if (slot > lim) x[r] = -INFINITY;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          const int slot = 32 * (r / 16) + 8 * ((r % 16) / 4) + 4 * hf + (r % 4);
          int key = INT_MAX;
          if (slot < cur.len) {
            key = cur.gathered ? cols[cur.base + slot] : cur.base + slot;
            if (!col_ok(key, N)) key = INT_MAX;
          }
          if (key > qpos) x[r] = -INFINITY;
        }
      }
    }
    // Block mode: the first half's probabilities are made with the current
    // reference before the maximum is known (the lazy rescale below rarely
    // moves it), so these exps overlap the second half's products; they are
    // redone if the reference moves.
    constexpr bool SPEC = (MODE == 0);
    const float mspec = (m == -INFINITY) ? 0.f : m;
    float xs[SPEC ? 16 : 1];
    if constexpr (SPEC) {
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[r] = fast_exp2(fmaf(x[r], sl2, -mspec));
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 32; ++r) mx = fmaxf(mx, x[r]);
    mx = xor32_max(mx) * sl2;
    // Lazy rescaling: the reference maximum m only moves when the tile's
    // maximum exceeds it by more than kSlack (log2 units), so probabilities
    // stay below 2^kSlack and O / l are rescaled only on such jumps.  The
    // final O / l and lse use the same m, so the result is exact up to rounding.
    if (__any(mx > m + kSlack)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
      if (__any(m != -INFINITY)) {
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      m = mnew;
    }
    const float muse = (m == -INFINITY) ? 0.f : m;
    if constexpr (SPEC) {
      if (__any(muse != mspec)) {  // the reference moved: redo the first half
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[r] = fast_exp2(fmaf(x[r], sl2, -muse));
      }
    }

    // ---- V(t) in LDS: the probabilities are made one k-step at a time, each
    //      step's P^T operand (8 consecutive registers x[8ks .. 8ks+7]) going
    //      straight into its products, so the exps of step ks+1 run on the VALU
    //      while the matrix core works on step ks
    if (more) wait_vmcnt<NDMA>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    // O^T += V^T . P^T; the A operand (dims 32dt + l32, keys 16ks + 4hf + e and
    // 16ks + 8 + 4hf + e) comes from two transposing reads: in each 16-lane group,
    // lane j points at V[key0 + j/4][dim0 + 4(j%4) .. +3]
    const int gl = lane & 15, gsub = (lane >> 4) & 1;
    float pp[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short dependency chains
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 pvk;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * ks + e;
        if (SPEC && r < 16) x[r] = xs[SPEC ? r : 0];
        else x[r] = fast_exp2(fmaf(x[r], sl2, -muse));
        pp[r & 3] += x[r];
        pvk[e] = (__bf16)x[r];
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {  // independent accumulators back to back
        const int dim = 32 * dt + 16 * gsub + 4 * (gl & 3);
        const int k0 = 16 * ks + 4 * hf + (gl >> 2);
        const int a0 = k0 * D + 8 * ((dim >> 3) ^ swz_key<D>(k0)) + (dim & 7);
        const int k1 = k0 + 8;
        const int a1 = k1 * D + 8 * ((dim >> 3) ^ swz_key<D>(k1)) + (dim & 7);
        const v4i16 lo = lds_read_tr16(Vl + a0);
        const v4i16 hi = lds_read_tr16(Vl + a1);
        const short __attribute__((ext_vector_type(8))) ab = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, ab), pvk, o[dt]);
      }
    }
    float ps = (pp[0] + pp[1]) + (pp[2] + pp[3]);
    ps = xor32_add(ps);
    lsum += ps;
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();  // both waves are done with V(t)
    if (more) dma_tile<D>(Vl, vb, nxt, cols, N, w, lane);
    cur = nxt;
    have = more;
  }

  // ---- epilogue: O = O^T / l, element (dt, r) is dim 32dt + 8(r/4) + 4hf + r%4
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int64_t orow = ((int64_t)b * p.heads_q + h) * N + qpos;
  if (OUT_BF16) {
    uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + orow * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 pk;
        pk[0] = pack_bf16x2(o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv);
        pk[1] = pack_bf16x2(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * j + 4 * hf) = pk;
      }
  } else {
    float* op = reinterpret_cast<float*>(p.out) + orow * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 v4;
        for (int e = 0; e < 4; ++e) v4[e] = o[dt][4 * j + e] * inv;
        *reinterpret_cast<f32x4*>(op + 32 * dt + 8 * j + 4 * hf) = v4;
      }
  }
  if (p.lse != nullptr && hf == 0) p.lse[orow] = lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ fp32 inputs
// One workgroup of 512 threads per (batch, head, query block): eight threads per
// query row, each owning an eighth of the head dimensions (fp32 throughout).
// Per 64-key tile a thread forms its partial dot products with the tile's keys,
// the row's eight partials are summed by three lane exchanges in a fixed order
// (so the eight threads hold identical scores), and the online softmax and the
// P.V products run on the thread's eighth of the output.
constexpr int kF32Threads = 512;

// X = 1 or 2: v + the value of lane l ^ X within each quad (DPP quad permute).
// X = 4: v + the value of lane 7 - l within each group of 8 (row_half_mirror),
// which after the two quad steps holds the other quad's sum.
template <int X>
__device__ __forceinline__ float quad_xor_add(float v) {
  constexpr int ctrl = X == 1 ? 0xB1 : (X == 2 ? 0x4E : 0x141);  // quad_perm [1,0,3,2] / [2,3,0,1] / row_half_mirror
  const int o = __builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false);
  return v + __int_as_float(o);
}

template <int D, int MODE>
__global__ __launch_bounds__(kF32Threads) void k_fwd_f32(FwdParams p) {
  constexpr int DQ = D / 8;  // dimensions per thread
  constexpr int C4 = D / 4;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) float Ks[kBlk][D];
  __shared__ __attribute__((aligned(16))) float Vs[kBlk][D];
  __shared__ int32_t keyS[kBlk];
  __shared__ int32_t ash[MODE == 0 ? 2048 : 1];
  const int tid = threadIdx.x, rw = tid >> 3, part = tid & 7;
  const Item item = item_at(p, blockIdx.x, gridDim.x, 0);
  const int b = item.b, h = item.h, iblk = item.iblk;
  const int g = h / (p.heads_q / p.heads_kv);
  const int64_t N = p.seq;
  const int64_t row_id = item.trow;
  const int qpos = iblk * kBlk + rw;
  const float* qr = reinterpret_cast<const float*>(p.q) + (((int64_t)b * p.heads_q + h) * N + qpos) * D + part * DQ;
  const float* kb = reinterpret_cast<const float*>(p.k) + ((int64_t)b * p.heads_kv + g) * N * D;
  const float* vb = reinterpret_cast<const float*>(p.v) + ((int64_t)b * p.heads_kv + g) * N * D;

  TileIter<MODE> it;
  const int32_t* cols = nullptr;
  if (MODE == 0) {
    if (p.ashape) {
      it.cnt = ashape_list(ash, iblk, p.n_sink, p.n_local, tid, kF32Threads);
      it.bidx = ash;
      __syncthreads();
    } else {
      it.bidx = p.block_idx + row_id * p.kmax;
      it.cnt = max(0, min(p.block_cnt[row_id], p.kmax));
    }
    it.iblk = iblk;
    it.start_blocks();
  } else {
    // the same clipping as the bf16 kernel: counts to capacities, intervals to
    // the keys the block can see, columns outside [0, seq) masked
    it.iv = p.iv + row_id * p.max_iv * 2;
    it.n_iv = max(0, min(p.iv_cnt[row_id], p.max_iv));
    it.n_col = max(0, min(p.col_cnt[row_id], p.max_col));
    it.iblk = iblk;
    it.lim = (int)min(N, (int64_t)iblk * kBlk + kBlk);
    it.bad_cols = 1;  // every gathered key is checked below anyway
    cols = p.col + row_id * p.max_col;
  }
  float q[DQ], o[DQ];
#pragma unroll
  for (int d = 0; d < DQ; d += 4) {
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(qr + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[d + e] = v4[e];
      o[d + e] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f;
  TileRef r;
  while (it.next(r)) {
    __syncthreads();  // the previous tile's K and V are no longer read
    for (int e = tid; e < kBlk * C4; e += kF32Threads) {
      const int slot = e / C4, c = e % C4;
      const int64_t row = tile_row(r, cols, slot, N);
      *reinterpret_cast<f32x4*>(&Ks[slot][4 * c]) = *reinterpret_cast<const f32x4*>(kb + row * D + 4 * c);
      *reinterpret_cast<f32x4*>(&Vs[slot][4 * c]) = *reinterpret_cast<const f32x4*>(vb + row * D + 4 * c);
    }
    if (tid < kBlk) {
      int key = INT_MAX;
      if (tid < r.len) {
        key = r.gathered ? cols[r.base + tid] : r.base + tid;
        if (!col_ok(key, N)) key = INT_MAX;
      }
      keyS[tid] = key;
    }
    __syncthreads();
    float s[kBlk];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < kBlk; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < DQ; d += 4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(&Ks[c][part * DQ + d]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(q[d + e], k4[e], acc);
      }
      acc = quad_xor_add<4>(quad_xor_add<2>(quad_xor_add<1>(acc)));  // ((p0 + p1) + (p2 + p3)) + (...) on all eight lanes
      s[c] = keyS[c] > qpos ? -INFINITY : acc * p.scale;
      mx = fmaxf(mx, s[c]);
    }
    const float mnew = fmaxf(m, mx);
    if (mnew == -INFINITY) continue;
    const float alpha = expf(m - mnew);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < DQ; ++d) o[d] *= alpha;
#pragma unroll
    for (int c = 0; c < kBlk; ++c) {
      const float pc = expf(s[c] - mnew);
      l += pc;
#pragma unroll
      for (int d = 0; d < DQ; d += 4) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(&Vs[c][part * DQ + d]);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[d + e] = fmaf(pc, v4[e], o[d + e]);
      }
    }
    m = mnew;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = ((int64_t)b * p.heads_q + h) * N + qpos;
  if (p.lse != nullptr && part == 0) p.lse[orow] = l > 0.f ? m + logf(l) : -INFINITY;
  float* op = reinterpret_cast<float*>(p.out) + orow * D + part * DQ;
#pragma unroll
  for (int d = 0; d < DQ; d += 4) {
    f32x4 v4 = {o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv};
    *reinterpret_cast<f32x4*>(op + d) = v4;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int head_dim, int mode, bool in_bf16, bool out_bf16,
                      hipStream_t stream) {
  const int n_items = p.batch * (p.hl.n > 0 ? p.hl.n : p.heads_q) * p.nqb;
  if (n_items == 0) return hipSuccess;
  const dim3 grid(n_items);
  // KV-head-major order once the K/V of all heads (bf16) outgrows ~192 MB,
  // i.e. no longer fits the Infinity Cache beside everything else.
  const double kv_bytes = 4.0 * p.batch * p.heads_kv * (double)p.seq * head_dim;
  FwdParams pp = p;
  pp.order = (in_bf16 && p.nqb % 64 == 0 && n_items % kXcds == 0 && kv_bytes > 192.0 * (1 << 20)) ? 1 : 0;
  if (in_bf16) {
#define SA_FWD_CASE(D_, M_, OB_)                                                   \
  if (head_dim == D_ && mode == M_ && out_bf16 == OB_) {                           \
    hipLaunchKernelGGL((k_fwd_bf16<D_, M_, OB_>), grid, dim3(kThreads), 0, stream, pp); \
    return hipGetLastError();                                                      \
  }
    SA_FWD_CASE(128, 0, true)
    SA_FWD_CASE(128, 0, false)
    SA_FWD_CASE(128, 1, true)
    SA_FWD_CASE(128, 1, false)
    SA_FWD_CASE(64, 0, true)
    SA_FWD_CASE(64, 0, false)
    SA_FWD_CASE(64, 1, true)
    SA_FWD_CASE(64, 1, false)
#undef SA_FWD_CASE
    return hipErrorInvalidValue;
  }
  if (out_bf16) return hipErrorInvalidValue;
#define SA_FWD32_CASE(D_, M_)                                                   \
  if (head_dim == D_ && mode == M_) {                                           \
    hipLaunchKernelGGL((k_fwd_f32<D_, M_>), grid, dim3(kF32Threads), 0, stream, p); \
    return hipGetLastError();                                                   \
  }
  SA_FWD32_CASE(64, 0)
  SA_FWD32_CASE(64, 1)
  SA_FWD32_CASE(128, 0)
  SA_FWD32_CASE(128, 1)
#undef SA_FWD32_CASE
  return hipErrorInvalidValue;
}

}  // namespace sa
