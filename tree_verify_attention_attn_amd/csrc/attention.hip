// attention.hip - tree-masked attention over a paged GQA KV cache (gfx950).
//
// What is computed (EAGLE-2 deep-dive page, third pillar; production note on
// indexing tree masks directly over paged memory): every tree node's query
// rows attend to the whole cached prefix of their sequence plus the tree
// positions whose bit is set in the node's ancestor mask.
//
// Work unit: one (sequence b, KV head g, row group, key split). The G query
// heads of a GQA group share the KV head, so the G*N (node, head) rows of a
// (b, g) pair form the query side of one dense product and each 64-key K/V
// tile is read from HBM once per row group, staged in LDS by LDS-DMA
// (buffer_load ... lds) through a four-stage ring per K and V, and shared by
// the workgroup's wavefronts (32 query rows each).
//
// Matrix cores: S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16
// d from LDS, B = 16 d x 32 queries held in VGPRs). In the 32x32 result a lane
// owns one query column and 16 of the 32 keys (rows 8i + 4*(lane/32) + j), so
// the softmax row reductions are in-lane plus one permlane32 swap. The same
// accumulator, packed to bf16, is the B operand of O^T = V^T . P^T; its A
// operand (32 d x 16 keys of V^T) comes from the row-major V tile through the
// LDS transpose read (ds_read_b64_tr_b16), so V is never transposed in memory.
// Softmax is online in base 2 with lazy rescaling: O and l are rescaled only
// when a row's running max grows by more than 2^8, which bounds p <= 256.
// Only tiles that reach the tree positions or the sequence tail evaluate the
// mask; prefix tiles never do.
//
// Schedule: the two halves of the workgroup share SIMDs (wavefront w and
// w + NW/2) and run the same code offset by one barrier, so while one half
// runs a tile's matrix products (X phase) the other runs the softmax of the
// previous tile (Y phase) on the vector ALU.
#include <math.h>

#include <type_traits>

#include "tv_internal.h"

namespace tv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kKeys = 64;      // keys per tile
constexpr int kLook = 6;      // X phase: fragment reads run this many products ahead
constexpr int kMaxChunkTiles = 256;  // tiles per key split (bounds the LDS copy of its page ids)
constexpr int kMinSplitTiles = 6;    // shorter sequences (in 64-key tiles) are never split
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;  // lazy-rescale threshold (log2 units)
// Split partials O/l go to HBM in fp16 when every element of the row is at
// most this large (fp16 then rounds each within 2^-12 * 4 < 1e-3), else in
// fp32: half the partial traffic in the common case, no range or precision
// limit in the others
constexpr float kHalfBound = 4.0f;
constexpr double kMallBytes = 256.0 * 1024 * 1024;  // the MI355X Infinity Cache

struct AttnArgs {
  const uint16_t *q, *k, *v;
  const int32_t *page_table, *prefix_lens;
  const uint64_t *mask;
  const int32_t *sizes;  // node count of each sequence, or null (all N)
  int W;                 // mask words per row, ceil(N / 64)
  int64_t num_pages;
  int maxp, max_prefix_len;
  int B, N, Hq, Hkv, G, rows, rows_pad;
  int row_groups;
  float c;         // |sm_scale| * log2(e)
  int negate_q;    // sm_scale < 0: negate Q (exact) and use |sm_scale|
  void *out;
  int out_bf16;
  uint16_t *ws_h;  // split partials O/l in fp16 [slot][D] (rows whose |O/l| stays within kHalfBound)
  float *ws_ml;    // (m, l) per slot; l is stored as -1 - l when the row's O/l went to ws_o
  float *ws_o;     // split partials O/l in fp32 [slot][D], for the other rows
  int S, chunk_tiles;
  int xcd_remap;   // block ids are laid out so one (b, g) stays on one XCD
  const int32_t *order;  // or null: workgroup i runs unit order[i] (one split, one row group)
  unsigned long long *state;
};

__device__ inline float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ inline float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ inline bf16x4 lds_read_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)((__attribute__((address_space(3))) uint16_t *)p));
}

__device__ inline void store_out(const AttnArgs &a, int64_t base, int d, const float *v4) {
  if (a.out_bf16) {
    uint16_t *o = static_cast<uint16_t *>(a.out) + base + d;
    uint2 pk;
    pk.x = float_to_bf16_bits(v4[0]) | (static_cast<uint32_t>(float_to_bf16_bits(v4[1])) << 16);
    pk.y = float_to_bf16_bits(v4[2]) | (static_cast<uint32_t>(float_to_bf16_bits(v4[3])) << 16);
    *reinterpret_cast<uint2 *>(o) = pk;
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + base + d) = make_float4(v4[0], v4[1], v4[2], v4[3]);
  }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over one KV page (all KV heads, `bytes` long): loads outside
// [0, bytes) return zeros, so an unused or invalid page costs no branch.
__device__ inline i32x4 page_rsrc(const uint16_t *base, int64_t pid, int page_elems, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base + pid * page_elems);
  i32x4 r;
  r[0] = static_cast<int>(p & 0xFFFFFFFFull);
  r[1] = static_cast<int>((p >> 32) & 0xFFFFull);  // stride 0
  r[2] = bytes;
  r[3] = 0x00020000;
  return r;
}

// 16-byte-per-lane load from a buffer straight into LDS: lane i's data lands
// at lds_addr + 16 i (the LDS address goes in M0, which the compiler sets
// from the operand). Issued as inline assembly so that the compiler does not
// serialise the multi-stage pipeline with conservative waits; completion is
// tracked by the explicit vmcnt waits in the tile loop. NT marks the load
// non-temporal (streamed, not kept in the caches): the form for calls whose
// K/V stream is larger than the 256 MB Infinity Cache, where nothing it would
// keep survives to the next call anyway.
template <bool NT>
__device__ inline void dma16(uint32_t lds_addr, int voff, i32x4 rsrc) {
  if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ inline void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// LDS chunk swizzle of key row r: 16-byte chunk c is stored at position
// c ^ swz(r). The gfx950 LDS has 64 four-byte banks (256 bytes per cycle);
// a 16-byte read is served 16 lanes per cycle and an 8-byte transpose read 32
// lanes per cycle. For the K fragment reads (16 consecutive rows, one chunk
// each) swz must spread 16 rows over all 64 banks; for the V^T transpose
// reads (4 consecutive rows x 4 consecutive chunks per 32 lanes) it must move
// each row's 64-byte group to its own banks. D = 128 (256-byte rows) and
// D = 64 (128-byte rows, two rows per bank sweep) need different bits.
template <int D>
__device__ inline int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ inline uint32_t lds_addr_of(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char *)p));
}

template <int D, int NW, int STAGES, bool FLAT, bool KSPLIT, bool NT>
__global__ void __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_mfma_kernel(AttnArgs a) {
  constexpr int KS = D / 16;             // 16-wide d steps of S^T = K Q^T
  constexpr int DB = D / 32;             // 32-wide d blocks of O^T
  constexpr int RB = D * 2;              // bytes per key row in LDS (no padding: rows are XOR-swizzled)
  constexpr int CPR = D / 8;             // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;          // key rows per 1 KB DMA instruction
  constexpr int IPW = CPR / NW;          // K (and V) DMA instructions per wavefront per tile
  constexpr int TILE_BYTES = kKeys * RB; // one K (or V) tile
  constexpr int ROWS_WG = KSPLIT ? 32 : 32 * NW;  // key split: every wavefront holds the same 32 rows
  constexpr int WROW = KSPLIT ? 0 : 32;          // row offset between wavefronts
  static_assert(!KSPLIT || NW == 2, "key split pairs two wavefronts");
  static_assert(IPW >= 1 && CPR % NW == 0, "workgroup too wide for the tile");

  // stage s: K tile at [s][0], V tile at [s][1]; rows are 2*D bytes with
  // swizzled chunk positions (see swz), conflict-free without padding
  __shared__ __align__(1024) uint8_t smem[STAGES][2][TILE_BYTES];
  __shared__ int s_bad;
  // this split's pages: their byte offsets in the pool (FLAT) or their ids
  __shared__ int s_pid[kMaxChunkTiles * (kKeys / kPage)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so DMA operands stay scalar
  const int h = lane >> 5, n = lane & 31;

  // block -> (b, g, row group, split); consecutive logical ids share an XCD
  int id = blockIdx.x;
  if (a.order)
    id = a.order[id];  // one workgroup per (b, g): the longest units are dispatched first
  else if (a.xcd_remap)
    id = (id & 7) * (gridDim.x >> 3) + (id >> 3);
  const int s = id % a.S;
  const int rg = (id / a.S) % a.row_groups;
  const int bh = id / (a.S * a.row_groups);
  const int b = bh / a.Hkv, g = bh % a.Hkv;

  // this split's page-table entries, read before the sequence's length and
  // node count are known so that the two reads overlap (entries past the
  // sequence's last page are dropped once the length is in; the read stays
  // inside the table's row). All of a thread's loads are issued at once.
  constexpr int kPidPerThread = kMaxChunkTiles * (kKeys / kPage) / (64 * NW);
  const int t_begin = s * a.chunk_tiles;
  const int64_t pt_row = static_cast<int64_t>(b) * a.maxp;
  int pid_in[kPidPerThread];
  {
    const int p0 = t_begin * (kKeys / kPage);
    const int avail = min(a.chunk_tiles * (kKeys / kPage), a.maxp - p0);
#pragma unroll
    for (int e = 0; e < kPidPerThread; ++e) {
      const int i = tid + e * 64 * NW;
      pid_in[e] = i < avail ? a.page_table[pt_row + p0 + i] : -1;
    }
  }

  const int L = a.prefix_lens[b];
  // node count of this sequence: nodes past it are absent (no query rows,
  // no keys); a count outside [1, N] is bad data, reported like a bad length
  const int nb_in = a.sizes ? a.sizes[b] : a.N;
  const bool bad_size = nb_in < 1 || nb_in > a.N;
  const int nb = bad_size ? a.N : nb_in;
  const int rows_b = nb * a.G;
  if (rg * ROWS_WG >= rows_b) return;  // every row of this workgroup is absent
  const bool bad_len = L < 0 || L > a.max_prefix_len || bad_size;
  const int T = bad_len ? 0 : L + nb;
  const int tiles_b = (T + kKeys - 1) / kKeys;
  const int t_end = min(t_begin + a.chunk_tiles, tiles_b);
  const int ntiles = max(t_end - t_begin, 0);
  if (tid == 0) s_bad = 0;

  // ---- the wavefront's 32 query rows: B operands of S^T, kept in VGPRs
  const int row = rg * ROWS_WG + w * WROW + n;
  const bool wave_active = rg * ROWS_WG + w * WROW < rows_b;
  const bool row_ok = row < rows_b;
  const int node = row_ok ? row / a.G : 0;
  const int head = g * a.G + (row_ok ? row % a.G : 0);
  // the row's ancestor mask over the present nodes: bits of nodes 0..63 in
  // mw0, of nodes 64..127 in mw1 (all present nodes when there is no mask)
  uint64_t mw0 = ~0ull, mw1 = ~0ull;
  if (row_ok && a.mask) {
    const int64_t mrow = (static_cast<int64_t>(b) * a.N + node) * a.W;
    mw0 = a.mask[mrow];
    mw1 = a.W > 1 ? a.mask[mrow + 1] : 0ull;
  }
  mw0 &= nb >= 64 ? ~0ull : ((1ull << nb) - 1ull);
  mw1 &= nb <= 64 ? 0ull : (nb >= 128 ? ~0ull : ((1ull << (nb - 64)) - 1ull));
  bf16x8 qf[KS];
  {
    const uint16_t *qrow = a.q + ((static_cast<int64_t>(b) * a.N + node) * a.Hq + head) * D;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *reinterpret_cast<const uint4 *>(qrow + 16 * t + 8 * h);
      if (a.negate_q) {
        v.x ^= 0x80008000u;
        v.y ^= 0x80008000u;
        v.z ^= 0x80008000u;
        v.w ^= 0x80008000u;
      }
      qf[t] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m_ref = -INFINITY, l = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;

  // ---- DMA. K tiles and V tiles have rings of their own (tile j of the
  // split uses stage j % STAGES of each). A tile's 16-byte chunks are moved
  // by 1 KB instructions: instruction jj covers key rows [jj*RPI, (jj+1)*RPI)
  // (inside one page) and lane i fills chunk position i % CPR of row
  // jj*RPI + i / CPR with logical chunk (i % CPR) ^ swz(row). Wavefront w
  // issues the IPW consecutive instructions jj = w*IPW + q, which share one
  // page whenever IPW*RPI <= 16, so a page id is looked up once per page.
  // FLAT: the whole K (and V) pool is below 2 GiB, so one buffer resource per
  // pool serves every page and the page's byte offset goes into the VGPR
  // offset; an invalid page or a key past the sequence gets an offset past
  // the resource's size, which loads zeros. Otherwise each page gets its own
  // resource (size 0 when the page id is invalid).
  constexpr int PPW = (IPW * RPI + kPage - 1) / kPage;  // pages per wavefront per tile
  const int page_elems = a.Hkv * kPage * D;
  const int page_bytes = page_elems * 2;
  const uint32_t npages32 = static_cast<uint32_t>(min(a.num_pages, static_cast<int64_t>(0x7FFFFFFF)));
  const uint32_t smem_base = lds_addr_of(&smem[0][0][0]);
  bool load_bad = false;
  int dma_off[IPW];  // byte offset of the lane's chunk inside its page (row slot, KV head, chunk)
#pragma unroll
  for (int q = 0; q < IPW; ++q) {
    const int r = (w * IPW + q) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(r);
    dma_off[q] = ((g * kPage + r % kPage) * D + c * 8) * 2;
  }
  const int lane_row = lane / CPR;
  i32x4 pool_rsrc[2];
  if constexpr (FLAT) {
    const int pool_bytes = static_cast<int>(a.num_pages * page_bytes);
    pool_rsrc[0] = page_rsrc(a.k, 0, 0, pool_bytes);
    pool_rsrc[1] = page_rsrc(a.v, 0, 0, pool_bytes);
  }
  // page entries (byte offsets or ids) of tile j for this wavefront, read
  // from LDS (the value is uniform; it is read ahead of the issue so that
  // the LDS latency is hidden)
  auto fetch = [&](int j, int (&pid)[PPW]) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PPW; ++p) pid[p] = s_pid[j * (kKeys / kPage) + (w * IPW * RPI) / kPage + p];
  };
  // A DMA item (tile j, part) is issued in three steps: fetch (LDS read of its
  // page entries, placed before a barrier so that its latency is hidden),
  // resolve (to wave-uniform page offsets, right after the barrier, when no
  // other LDS read is outstanding, so the wait for the read is free) and
  // issue_range (the DMA instructions, spread over the phase; no waits).
  struct DmaItem {
    int j, part, poff[PPW];
    bool on;
  };
  auto resolve = [&](int j, int part, bool on, const int (&pidv)[PPW]) __attribute__((always_inline)) {
    DmaItem it;
    it.j = j;
    it.part = part;
    it.on = on;
    if (on) {
      const int tile0 = (t_begin + j) * kKeys;
#pragma unroll
      for (int p = 0; p < PPW; ++p) {
        const int pid = __builtin_amdgcn_readfirstlane(pidv[p]);
        if constexpr (FLAT) {
          it.poff[p] = pid;  // already the byte offset (bad pages were found in the prologue)
        } else {
          const bool ok = static_cast<uint32_t>(pid) < npages32;
          if (part == 0) load_bad |= (tile0 + w * IPW * RPI + p * kPage < T) && !ok;
          it.poff[p] = ok ? pid : -1;
        }
      }
    }
    return it;
  };
  // instructions [q0, q1) of this wavefront's share of an item
  auto issue_range = [&](const DmaItem &it, int q0, int q1) __attribute__((always_inline)) {
    if (!it.on) return;
    const int tile0 = (t_begin + it.j) * kKeys;
    const int row0 = w * IPW * RPI;  // first key row of this wavefront's instructions
    const bool full = tile0 + row0 + IPW * RPI <= T;
    const uint32_t dst0 = smem_base + ((it.j % STAGES) * 2 + it.part) * TILE_BYTES + w * IPW * 1024;
    if constexpr (FLAT) {
      if (full) {  // every key row of this wavefront's share is inside the sequence
#pragma unroll
        for (int q = 0; q < IPW; ++q) {
          if (q < q0 || q >= q1) continue;
          dma16<NT>(dst0 + q * 1024, it.poff[q * PPW / IPW] + dma_off[q], pool_rsrc[it.part]);
        }
        return;
      }
    }
#pragma unroll
    for (int q = 0; q < IPW; ++q) {
      if (q < q0 || q >= q1) continue;
      const int p = q * PPW / IPW;  // page of instruction q
      if constexpr (FLAT) {
        int voff = it.poff[p] + dma_off[q];
        if (!full && tile0 + row0 + q * RPI + lane_row >= T) voff = static_cast<int>(0x80000000u);
        dma16<NT>(dst0 + q * 1024, voff, pool_rsrc[it.part]);
      } else {
        const bool ok = it.poff[p] >= 0;
        int voff = dma_off[q];
        if (!full && tile0 + row0 + q * RPI + lane_row >= T) voff = 0x7FFFFFF0;
        dma16<NT>(dst0 + q * 1024, voff,
              page_rsrc(it.part ? a.v : a.k, ok ? it.poff[p] : 0, page_elems, ok ? page_bytes : 0));
      }
    }
  };
  auto issue_now = [&](int j, int part) __attribute__((always_inline)) {
    int pid[PPW];
    fetch(j, pid);
    issue_range(resolve(j, part, true, pid), 0, IPW);
  };

  // this split's pages, copied once into LDS so that the DMA issue path never
  // waits on a memory round trip: with one resource per pool as byte offsets
  // (past the resource for a page past the sequence's end or outside the
  // pool), and the workgroup learns here whether the sequence has a bad page;
  // otherwise as page ids (-1 past the sequence's end)
  {
    const int p0 = t_begin * (kKeys / kPage);
    const int used = min(t_end * (kKeys / kPage), (T + kPage - 1) / kPage) - p0;
    int bad_here = 0;
#pragma unroll
    for (int e = 0; e < kPidPerThread; ++e) {
      const int i = tid + e * 64 * NW;
      if (i < ntiles * (kKeys / kPage)) {
        if constexpr (FLAT) {
          // the page's byte offset in the pool, or an offset past the pool's
          // resource (loads of zeros) for a page outside the pool or past the
          // sequence; a page inside the sequence that is not in the pool is bad
          const bool ok = static_cast<uint32_t>(pid_in[e]) < npages32;
          bad_here |= i < used && !ok;
          s_pid[i] = i < used && ok ? pid_in[e] * page_bytes : static_cast<int>(0x80000000u);
        } else {
          s_pid[i] = i < used ? pid_in[e] : -1;
        }
      }
    }
    if constexpr (FLAT)
      load_bad = __syncthreads_or(bad_here) != 0;
    else
      __syncthreads();
  }

  // per-lane LDS byte offsets of the fragment reads (swizzled chunk positions)
  int koff[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) koff[t] = n * RB + (((2 * t + h) ^ swz<D>(n)) << 4);
  // V^T transpose read: lane (group grp, slot sl) addresses key row
  // 4h + sl/4 (+16 m2, +8, +32 kb) and d 32 db + 16 (grp % 2) + 4 (sl % 4)
  const int grp = lane >> 4, sl = lane & 15;
  const int vr = 4 * h + (sl >> 2);  // key row (within 16) of the low half; the high half reads vr + 8
  int voff_lo[DB], voff_hi[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int c = 4 * db + 2 * (grp & 1) + ((sl & 3) >> 1);
    voff_lo[db] = vr * RB + ((c ^ swz<D>(vr)) << 4) + ((sl & 1) << 3);
    voff_hi[db] = (vr + 8) * RB + ((c ^ swz<D>(vr + 8)) << 4) + ((sl & 1) << 3);
  }

  auto kread = [&](int st, int kb, int t) -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(&smem[st][0][0] + kb * 32 * RB + koff[t]);
  };
  // V^T fragment (db, f) of a tile, f = 2 kb + m2 (32-key block kb, 16-key
  // half m2), is two transpose reads (keys +0 and +8)
  auto vread = [&](int st, int db, int f, int half) -> bf16x4 {
    const uint8_t *vb = &smem[st][1][0] + ((f >> 1) * 32 + 16 * (f & 1)) * RB;
    return lds_read_tr16(reinterpret_cast<const uint16_t *>(vb + (half ? voff_hi[db] : voff_lo[db])));
  };

  f32x16 sc[2];     // S_j^T (two 32-key blocks), from the X phase of tile j to its Y phase
  bf16x8 pk[2][2];  // P_j in bf16, from the Y phase of tile j to the X phase of tile j + 1

  // X phase of tile j (matrix cores): when j > 0, O += V_{j-1}^T P_{j-1}^T,
  // then S_j = K_j Q^T. PV goes first so that P_{j-1} is dead before S_j is
  // born. The products form one unrolled stream (16 PV, then 16 S at
  // D = 128); the A-operand fragment of product m is read from LDS kLook
  // products ahead, one read group per product: at most about 12 LDS reads
  // are in flight, so each product waits only for its own fragment (with
  // more than the 4-bit LDS counter's 15 reads outstanding, or a different
  // count on different paths into the phase, the wait would be for all of
  // them). The four O chains and the two S chains alternate, so
  // no MFMA waits on the one before it. For j == n the S products read a
  // stale stage; their result is never used.
  auto X = [&](int j, int jp) __attribute__((always_inline)) {
    const int ks = j % STAGES, vs = (jp + STAGES) % STAGES;
    constexpr int NPV = 4 * DB;  // PV products: 16-key step f, 32-d block db
    constexpr int NS = 2 * KS;   // S products: 16-d step t, 32-key block kb
    constexpr int LA = kLook;
    // A operand of product m (m < NPV: V^T fragment, two transpose reads;
    // else a K fragment, one 16-byte read)
    auto frag = [&](int m) __attribute__((always_inline)) -> bf16x8 {
      if (m < NPV) {
        const int f = m / DB, db = m % DB;
        return __builtin_shufflevector(vread(vs, db, f, 0), vread(vs, db, f, 1), 0, 1, 2, 3, 4, 5, 6, 7);
      }
      return kread(ks, (m - NPV) & 1, (m - NPV) >> 1);
    };
    auto product = [&](int m, const bf16x8 &a) __attribute__((always_inline)) {
      if (m < NPV) {
        const int f = m / DB, db = m % DB;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[f >> 1][f & 1], o[db], 0, 0, 0);
      } else {
        const int kb = (m - NPV) & 1, t = (m - NPV) >> 1;
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], sc[kb], 0, 0, 0);
      }
    };
    auto run = [&](auto m0c) __attribute__((always_inline)) {
      constexpr int M0 = decltype(m0c)::value;
      constexpr int NM = NPV + NS - M0;
      bf16x8 ring[LA];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        ring[i] = frag(M0 + i);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        bf16x8 nx;
        if (i + LA < NM) nx = frag(M0 + i + LA);
        product(M0 + i, ring[i % LA]);
        if (i + LA < NM) ring[i % LA] = nx;
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (jp >= 0)
      run(std::integral_constant<int, 0>());
    else
      run(std::integral_constant<int, NPV>());
  };

  // Y phase of tile j (vector ALU): tree/tail visibility, running max, lazy
  // rescale, exponentials, row sums and the bf16 P_j for the next X phase.
  // `mid(0)` runs after the row max and `mid(1)` halfway through the
  // exponentials (the DMA issue of the wavefronts whose turn it is).
  auto Y = [&](int j, auto &&mid) __attribute__((always_inline)) {
    const int tile0 = (t_begin + j) * kKeys;
    // visibility (only tiles that reach the tree positions or the tail): one
    // 64-bit word per tile, bit k = key tile0 + k is visible to this row
    if (tile0 + kKeys > L) {
      // key k of the tile is tree node off + k (-64 < off < nb): the 64-bit
      // window of the row's 128-bit ancestor mask that starts at node off
      const int off = tile0 - L;
      uint64_t tree;
      if (off < 0)
        tree = mw0 << -off;
      else if (off == 0)
        tree = mw0;
      else if (off < 64)
        tree = (mw0 >> off) | (mw1 << (64 - off));
      else if (off == 64)
        tree = mw1;
      else
        tree = mw1 >> (off - 64);
      const int pre = L - tile0;  // keys k < pre belong to the prefix
      const uint64_t prefix = pre <= 0 ? 0ull : ((1ull << pre) - 1ull);
      const uint64_t vis64 = prefix | tree;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t vb = static_cast<uint32_t>(vis64 >> (kb * 32 + 4 * h));
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sc[kb][e] = ((vb >> (8 * (e >> 2) + (e & 3))) & 1u) ? sc[kb][e] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
    mx = swap_halves_max(mx);
    const float mt = mx == -INFINITY ? -INFINITY : mx * a.c;
    // lazy rescale: only when some row's max grows by more than 2^kRescale
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + kRescale) != 0ull) {
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      m_ref = m_new;
    }
    const float mu = m_ref == -INFINITY ? 0.f : m_ref;
    mid(0);
    // masked scores are -inf and c > 0, so their p is exactly 0. P_j is built
    // in fresh vectors: element inserts into pk itself would keep P_{j-1}
    // live through this phase.
    bf16x8 np[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb == 1) mid(1);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][e], a.c, -mu));
        l += p;
        np[kb][e >> 3][e & 7] = static_cast<__bf16>(p);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      pk[kb][0] = np[kb][0];
      pk[kb][1] = np[kb][1];
    }
  };

  // Writes this wavefront's rows: the outputs (one split) or the split's
  // partial (o, m, l). With `nan` the outputs, or the partial's m, are NaN:
  // the workgroup met bad data. Every lane of the wavefront takes part (the
  // row sum's half swap).
  auto emit = [&](bool nan) __attribute__((always_inline)) {
    const float l_tot = swap_halves_sum(l);
    // the row's largest |O| (both halves of the wavefront take part)
    float amax = 0.f;
    if (a.S > 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(o[db][e]));
      amax = swap_halves_max(amax);
    }
    if (!row_ok) return;
    if (a.S == 1) {
      const int64_t base = ((static_cast<int64_t>(b) * a.N + node) * a.Hq + head) * D;
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = nan ? NAN : o[db][4 * i + j] * inv;
          store_out(a, base, db * 32 + 8 * i + 4 * h, v4);
        }
    } else {
      const int64_t slot = (static_cast<int64_t>(bh) * a.S + s) * a.rows_pad + row;
      // the partial is O/l (0 for a row with nothing visible in this split)
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const bool half = amax * inv <= kHalfBound;  // false for inf or NaN too
      if (half) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
            f16x4 hv;
#pragma unroll
            for (int j = 0; j < 4; ++j) hv[j] = static_cast<_Float16>(o[db][4 * i + j] * inv);
            *reinterpret_cast<f16x4 *>(a.ws_h + slot * D + db * 32 + 8 * i + 4 * h) = hv;
          }
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<float4 *>(a.ws_o + slot * D + db * 32 + 8 * i + 4 * h) =
                make_float4(o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                            o[db][4 * i + 3] * inv);
      }
      if (h == 0) {
        a.ws_ml[slot * 2] = nan ? NAN : m_ref;
        a.ws_ml[slot * 2 + 1] = half ? l_tot : -1.f - l_tot;
      }
    }
  };
  bool emitted = false, emitted_nan = false;

  if constexpr (KSPLIT) {
    // Key split (row groups of at most 32 rows): wavefront w takes tiles
    // w, w + 2, w + 4, ... of the split with its own running max, sum and O,
    // so both SIMDs of the workgroup compute. Iteration i holds tiles 2i and
    // 2i+1; after its barrier it refills K for tiles 2i+2, 2i+3 (the stages
    // of tiles 2i-2, 2i-1, read in iteration i-1) and V for tiles 2i, 2i+1
    // (read by the PV products of iteration i+1), and each iteration waits
    // for all of the previous one's DMA.
    const int n_t = ntiles;
    const int npairs = (n_t + 1) / 2;
    auto noop = [](int) {};
    if (n_t > 0) issue_now(0, 0);
    if (n_t > 1) issue_now(1, 0);
    for (int i = 0; i <= npairs; ++i) {
      wait_vmcnt<0>();
      barrier_only();
      if (2 * i + 2 < n_t) issue_now(2 * i + 2, 0);
      if (2 * i + 3 < n_t) issue_now(2 * i + 3, 0);
      if (2 * i < n_t) issue_now(2 * i, 1);
      if (2 * i + 1 < n_t) issue_now(2 * i + 1, 1);
      const int j = 2 * i + w, jp = j - 2;
      if (wave_active && (j < n_t || (jp >= 0 && jp < n_t))) {
        X(j, jp);  // for j >= n only the PV products of tile jp matter
        if (j < n_t) Y(j, noop);
      }
    }
  } else {
  // Ping-pong tile loop. Wavefront w and w + NW/2 share a SIMD; the two
  // halves of the workgroup run the same code, a Y phase and an X phase per
  // tile with a barrier after each, but the second half starts one barrier
  // late. Half-step h (between barriers h-1 and h) thus holds the first
  // half's Y(k-1) and the second half's X(k-1) when h = 2k, and the first
  // half's X(k) and the second half's Y(k-1) when h = 2k+1: one half's
  // matrix products always overlap the other half's exponentials.
  //   K_j is read at half-steps 2j+1 and 2j+2, V_j (by PV) at 2j+3 and 2j+4,
  //   and each ring has four stages. All DMA is issued from Y phases, where
  //   it does not stall the matrix products: during its Y phase of iteration
  //   k the first half (half-step 2k) refills its share of K_{k+2} and
  //   V_{k+1}, the second half (half-step 2k+1) its share of K_{k+3} and
  //   V_{k+2}. Both land at least five half-steps before their first use,
  //   and each half waits for its own group of two iterations back before
  //   the odd half-steps.
  const int n_t = ntiles;
  const bool first = w < NW / 2;  // wave-uniform
  const int lead = first ? 0 : 1;
  auto parts = [&](int j) { return j >= 0 && j < n_t ? IPW : 0; };
  // DMA instructions of this wavefront issued after its group holding K_j
  // and V_{j-1} (what half-step 2j+1 needs) and before that half-step
  auto wait_for = [&](int j) __attribute__((always_inline)) {
    if (j >= 0 && j + 2 < n_t) {  // every group of the last two iterations is in flight
      wait_vmcnt<4 * IPW>();
      return;
    }
    switch ((parts(j + 1) + parts(j) + parts(j + 2) + parts(j + 1)) / IPW) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<IPW>(); break;
      case 2: wait_vmcnt<2 * IPW>(); break;
      case 3: wait_vmcnt<3 * IPW>(); break;
      default: wait_vmcnt<4 * IPW>(); break;
    }
  };
  // prologue, in issue order: K_0 | K_1 V_0 (| K_2 V_1 for the second half)
  if (n_t > 0) issue_now(0, 0);
  if (n_t > 1) issue_now(1, 0);
  if (n_t > 0) issue_now(0, 1);
  if (!first) {
    if (n_t > 2) issue_now(2, 0);
    if (n_t > 1) issue_now(1, 1);
    wait_for(0);
    barrier_only();
  }
  int pid_k[PPW], pid_v[PPW];
  if (2 + lead < n_t) fetch(2 + lead, pid_k);
  if (1 + lead < n_t) fetch(1 + lead, pid_v);
  for (int k = 0; k <= n_t; ++k) {
    const int kt = k + 2 + lead, vt = k + 1 + lead;  // tiles refilled in this Y phase
    const DmaItem kit = resolve(kt, 0, kt < n_t, pid_k);
    const DmaItem vit = resolve(vt, 1, vt < n_t, pid_v);
    auto ystep = [&](int i) __attribute__((always_inline)) { issue_range(i == 0 ? kit : vit, 0, IPW); };
    if (k >= 1 && wave_active) {
      Y(k - 1, ystep);
    } else {
      ystep(0);
      ystep(1);
    }
    if (first) wait_for(k);
    barrier_only();
    // page ids for the next Y phase, read unconditionally (a clamped index;
    // the value is used only when that tile exists) so that the LDS reads
    // in flight are the same on every path
    fetch(min(kt + 1, kMaxChunkTiles - 1), pid_k);
    fetch(min(vt + 1, kMaxChunkTiles - 1), pid_v);
    if (wave_active && n_t > 0) X(k, k - 1);
    if (!first) wait_for(k + 1);
    barrier_only();
  }
  // The first half ran its last products one half-step before the second
  // half: it writes its rows while the second half finishes. If another
  // wavefront turns out to have met bad data, the rows are marked again below.
  if (first && wave_active) {
    emitted_nan = bad_len || load_bad;
    emit(emitted_nan);
    emitted = true;
  }
  if (first) barrier_only();
  }
  if (load_bad) s_bad = 1;
  __syncthreads();
  const bool bad = bad_len || s_bad;
  if (bad && tid == 0) raise_error(a.state, TV_ERR_INVALID_ARG);
  if constexpr (KSPLIT) {
    // merge wavefront 1's (m, l, O) into wavefront 0's through LDS (the tile
    // ring is idle now: every DMA was waited for and every read is done)
    float *xch = reinterpret_cast<float *>(&smem[0][0][0]);
    if (w == 1 && wave_active) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) xch[(db * 16 + e) * 64 + lane] = o[db][e];
      xch[DB * 16 * 64 + lane] = m_ref;
      xch[(DB * 16 + 1) * 64 + lane] = l;
    }
    __syncthreads();
    if (w == 1) return;
    if (wave_active) {
      const float m1 = xch[DB * 16 * 64 + lane], l1 = xch[(DB * 16 + 1) * 64 + lane];
      const float mm = fmaxf(m_ref, m1);
      const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = o[db][e] * a0 + xch[(db * 16 + e) * 64 + lane] * a1;
      l = l * a0 + l1 * a1;
      m_ref = mm;
    }
  }
  if (!wave_active) return;
  if (!emitted || (bad && !emitted_nan)) emit(bad);
}

// Merges the S partials (m, l, O/l) of each row in a fixed split order: the
// output is sum_s e^(m_s - M) l_s (O/l)_s / sum_s e^(m_s - M) l_s. A row is
// D/8 lanes, each owning eight consecutive d (one 16-byte fp16 load per
// partial, two 16-byte fp32 loads for the rare rows kept wide), so a
// wavefront holds 64*8/D rows. Partials are read eight splits at a time with
// every load of a batch issued before any is used; the running maximum is
// raised between batches (one batch when S <= 8, which is then the plain
// max-then-sum merge). The rows of one (b, g) run on the XCD whose L2 took
// that unit's partials.
template <int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a) {
  constexpr int LPR = D / 8;     // lanes per row, eight d each
  constexpr int RPW = 64 / LPR;  // rows per wavefront
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63, sub = lane % LPR;
  int64_t blk = blockIdx.x;
  if (a.xcd_remap && (gridDim.x & 7) == 0) blk = (blk & 7) * (gridDim.x >> 3) + (blk >> 3);
  const int64_t r = (blk * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  if (r >= static_cast<int64_t>(a.B) * a.Hkv * a.rows) return;
  const int bh = static_cast<int>(r / a.rows), row = static_cast<int>(r % a.rows);
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  const int nb_in = a.sizes ? a.sizes[b] : a.N;
  const int nb = (nb_in < 1 || nb_in > a.N) ? a.N : nb_in;
  if (row >= nb * a.G) return;  // an absent node's row has no output
  const int64_t slot0 = static_cast<int64_t>(bh) * a.S * a.rows_pad + row;
  float M = -INFINITY, lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  for (int s0 = 0; s0 < a.S; s0 += kBatch) {
    float2 ml[kBatch];
    f16x8 hv[kBatch];
    float ov[kBatch][8];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      ml[q] = make_float2(-INFINITY, 0.f);
      hv[q] = f16x8{};
      if (s0 + q < a.S) {
        const int64_t slot = slot0 + static_cast<int64_t>(s0 + q) * a.rows_pad;
        ml[q] = *reinterpret_cast<const float2 *>(a.ws_ml + slot * 2);
        hv[q] = *reinterpret_cast<const f16x8 *>(a.ws_h + slot * D + 8 * sub);
      }
    }
    // O/l of each split: fp16, or fp32 for the rows the split kept wide
    // (marked by a negative l; rare, so their second read is taken apart)
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[q][e] = static_cast<float>(hv[q][e]);
      if (ml[q].y < 0.f) {
        const int64_t slot = slot0 + static_cast<int64_t>(s0 + q) * a.rows_pad;
        const float4 lo = *reinterpret_cast<const float4 *>(a.ws_o + slot * D + 8 * sub);
        const float4 hi = *reinterpret_cast<const float4 *>(a.ws_o + slot * D + 8 * sub + 4);
        ov[q][0] = lo.x; ov[q][1] = lo.y; ov[q][2] = lo.z; ov[q][3] = lo.w;
        ov[q][4] = hi.x; ov[q][5] = hi.y; ov[q][6] = hi.z; ov[q][7] = hi.w;
        ml[q].y = -1.f - ml[q].y;
      }
    }
    float Mb = M;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      bad |= isnan(ml[q].x);
      Mb = fmaxf(Mb, ml[q].x);
    }
    if (Mb != M) {  // raise the running maximum (M = -inf holds nothing yet)
      const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
      lsum *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= sc;
      M = Mb;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      // weight of the split's O/l: e^(m - M) * l
      const float wgt = ml[q].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[q].x - M) * ml[q].y;
      lsum += wgt;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wgt, ov[q][e], acc[e]);
    }
  }
  const int i = row / a.G, h = g * a.G + row % a.G;
  const int64_t base = ((static_cast<int64_t>(b) * a.N + i) * a.Hq + h) * D;
  const float inv = 1.f / lsum;
  float v4[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  float w4[4] = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  if (bad) v4[0] = v4[1] = v4[2] = v4[3] = w4[0] = w4[1] = w4[2] = w4[3] = NAN;
  store_out(a, base, 8 * sub, v4);
  store_out(a, base, 8 * sub + 4, w4);
}

// Orders the (b, g) units of a one-split plan by their number of 64-key tiles,
// longest first, so that a batch with very different prefix lengths does not
// end on its longest units (workgroups are dispatched in block order). One
// workgroup: a counting sort over tile counts (clamped to kOrderBuckets - 1).
// Only the schedule changes; every unit computes the same result.
constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = kOrderThreads;

__global__ void __launch_bounds__(kOrderThreads) order_units_kernel(const int32_t *__restrict__ prefix_lens,
                                                                    const int32_t *__restrict__ sizes, int B, int N,
                                                                    int Hkv, int max_prefix_len,
                                                                    int32_t *__restrict__ order) {
  __shared__ int s_cnt[kOrderBuckets];
  __shared__ int s_wsum[kOrderThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  auto bucket = [&](int b) {  // bucket 0 holds the most tiles
    const int L = prefix_lens[b];
    const int nb_in = sizes ? sizes[b] : N;
    const bool bad = L < 0 || L > max_prefix_len || nb_in < 1 || nb_in > N;
    const int t = bad ? 0 : (L + nb_in + 63) / 64;
    return kOrderBuckets - 1 - min(t, kOrderBuckets - 1);
  };
  s_cnt[tid] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kOrderThreads) atomicAdd(&s_cnt[bucket(b)], 1);
  __syncthreads();
  // exclusive scan of the bucket counts: within each wavefront, then over
  // the wavefront totals
  const int c = s_cnt[tid];
  int incl = c;
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  if (lane == 63) s_wsum[tid >> 6] = incl;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < (tid >> 6); ++i) off += s_wsum[i];
  s_cnt[tid] = off + incl - c;
  __syncthreads();
  for (int b = tid; b < B; b += kOrderThreads) {
    const int64_t pos = atomicAdd(&s_cnt[bucket(b)], 1);
    for (int g = 0; g < Hkv; ++g) order[pos * Hkv + g] = b * Hkv + g;
  }
}

constexpr int kStages = 4;

template <int D, bool FLAT, bool NT>
void launch_w(int qb, bool ksplit, dim3 grid, dim3 block, hipStream_t st, const AttnArgs &a) {
  if (ksplit)
    hipLaunchKernelGGL((attn_mfma_kernel<D, 2, kStages, FLAT, true, NT>), grid, block, 0, st, a);
  else if (qb == 8)
    hipLaunchKernelGGL((attn_mfma_kernel<D, 8, kStages, FLAT, false, NT>), grid, block, 0, st, a);
  else if (qb == 4)
    hipLaunchKernelGGL((attn_mfma_kernel<D, 4, kStages, FLAT, false, NT>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<D, 2, kStages, FLAT, false, NT>), grid, block, 0, st, a);
}

template <int D>
void launch_dw(int qb, bool ksplit, bool flat, bool nt, dim3 grid, dim3 block, hipStream_t st, const AttnArgs &a) {
  if (flat)
    nt ? launch_w<D, true, true>(qb, ksplit, grid, block, st, a) : launch_w<D, true, false>(qb, ksplit, grid, block, st, a);
  else
    nt ? launch_w<D, false, true>(qb, ksplit, grid, block, st, a)
       : launch_w<D, false, false>(qb, ksplit, grid, block, st, a);
}

}  // namespace

AttnPlan plan_attention(int cu_count, int B, int N, int Hq, int Hkv, int D, int max_prefix_len) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int rows = G * N;
  // 32 query rows per wavefront; 8, 4 or 2 wavefronts per workgroup
  p.qb = rows > 128 ? 8 : (rows > 64 ? 4 : 2);
  // up to 32 rows: two wavefronts share the rows and split the tiles
  p.ksplit = rows <= 32 ? 1 : 0;
  p.row_block = p.ksplit ? 32 : 32 * p.qb;
  p.row_blocks = (rows + p.row_block - 1) / p.row_block;
  const int tiles = (max_prefix_len + N + kKeys - 1) / kKeys;
  const int64_t base = static_cast<int64_t>(B) * Hkv * p.row_blocks;
  // about one workgroup per CU (LDS: two K/V tile buffers per workgroup)
  const int64_t target = static_cast<int64_t>(cu_count) * (p.qb == 8 ? 1 : 2);
  int64_t S = base > 0 ? (target + base / 2) / base : 1;
  if (S < 1) S = 1;
  if (S > tiles) S = tiles;
  // a short sequence is not split: below kMinSplitTiles tiles the partials
  // and the combine pass cost more than the tiles a split takes off the
  // longest workgroup (one sequence, 15 nodes, 4 heads: 3 tiles 13.2 us
  // unsplit against 16.1 us in three splits; 9 tiles 21.1 us unsplit against
  // 15.9 us in three splits)
  if (tiles < kMinSplitTiles) S = 1;
  if (S < (tiles + kMaxChunkTiles - 1) / kMaxChunkTiles) S = (tiles + kMaxChunkTiles - 1) / kMaxChunkTiles;
  if (S < 1) S = 1;
  p.chunk_tiles = static_cast<int>((tiles + S - 1) / S);
  if (p.chunk_tiles < 1) p.chunk_tiles = 1;
  p.S = (tiles + p.chunk_tiles - 1) / p.chunk_tiles;
  if (p.S < 1) p.S = 1;
  // per partial slot: O/l in fp16 and in fp32 (one of the two is written),
  // and (m, l)
  p.ws_bytes = p.S > 1 ? static_cast<size_t>(B) * Hkv * p.S * p.row_blocks * p.row_block *
                             (D * sizeof(uint16_t) + D * sizeof(float) + 2 * sizeof(float))
                       : 0;
  // many one-workgroup units (the key-split shape: short rows, many
  // sequences) whose prefix lengths may differ: dispatch the longest first
  p.order = (p.ksplit && p.S == 1 && base > cu_count) ? 1 : 0;
  // K/V loads marked non-temporal when the call's K/V stream (at the longest
  // prefix) exceeds the 256 MB Infinity Cache
  const double kv_bytes = static_cast<double>(B) * Hkv * (static_cast<double>(max_prefix_len) + N) * D * 2.0 * 2.0;
  p.nt = kv_bytes > kMallBytes ? 1 : 0;
  if (p.order) p.ws_bytes = static_cast<size_t>(B) * Hkv * sizeof(int32_t);
  return p;
}

tv_status launch_attention(tv_ctx *ctx, const AttnPlan &plan, const void *q, const void *k_pages,
                           const void *v_pages, int64_t num_pages, const int32_t *page_table, int maxp,
                           const int32_t *prefix_lens, int max_prefix_len, const uint64_t *tree_mask,
                           const int32_t *tree_sizes, int B, int N, int Hq, int Hkv, int D, float sm_scale, void *out,
                           tv_dtype out_dtype, void *workspace) {
  AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k_pages);
  a.v = static_cast<const uint16_t *>(v_pages);
  a.page_table = page_table;
  a.prefix_lens = prefix_lens;
  a.mask = tree_mask;
  a.sizes = tree_sizes;
  a.W = (N + 63) / 64;
  a.num_pages = num_pages;
  a.maxp = maxp;
  a.max_prefix_len = max_prefix_len;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.rows = a.G * N;
  a.rows_pad = plan.row_blocks * plan.row_block;
  a.row_groups = plan.row_blocks;
  // c > 0 keeps exp2(-inf * c) = 0 for masked keys; a zero scale becomes a
  // negligible positive one (every score then rounds to the same value)
  a.c = fmaxf(fabsf(sm_scale) * kLog2e, 1e-30f);
  a.negate_q = sm_scale < 0.f;
  a.out = out;
  a.out_bf16 = out_dtype == TV_BF16;
  a.S = plan.S;
  a.chunk_tiles = plan.chunk_tiles;
  a.state = ctx->d_state;
  if (plan.S > 1) {
    const int64_t slots = static_cast<int64_t>(B) * Hkv * plan.S * a.rows_pad;
    a.ws_h = static_cast<uint16_t *>(workspace);
    a.ws_ml = reinterpret_cast<float *>(a.ws_h + slots * D);
    a.ws_o = a.ws_ml + slots * 2;
  }
  const int blocks = B * Hkv * plan.row_blocks * plan.S;
  a.xcd_remap = (blocks % 8) == 0;
  if (plan.order) {
    a.order = static_cast<const int32_t *>(workspace);
    hipLaunchKernelGGL(order_units_kernel, dim3(1), dim3(kOrderThreads), 0, ctx->stream, prefix_lens, tree_sizes, B,
                       N, Hkv, max_prefix_len, static_cast<int32_t *>(workspace));
    if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  }
  const dim3 grid(blocks);
  const dim3 block(64 * plan.qb);
  // one buffer resource per pool when the pool is below 2 GiB (page offsets
  // then fit the 32-bit VGPR offset with room for the out-of-range marker)
  const bool flat = num_pages * static_cast<int64_t>(Hkv) * kPage * D * 2 <= 0x7FFF0000LL;
  if (D == 128)
    launch_dw<128>(plan.qb, plan.ksplit, flat, plan.nt, grid, block, ctx->stream, a);
  else
    launch_dw<64>(plan.qb, plan.ksplit, flat, plan.nt, grid, block, ctx->stream, a);
  if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  if (plan.S > 1) {
    const int rows_per_wg = 4 * (64 / (D / 8));  // four wavefronts, 64*8/D rows each
    const dim3 cgrid(static_cast<unsigned>((static_cast<int64_t>(B) * Hkv * a.rows + rows_per_wg - 1) / rows_per_wg));
    if (D == 128)
      hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, dim3(256), 0, ctx->stream, a);
    else
      hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, dim3(256), 0, ctx->stream, a);
    if (hipGetLastError() != hipSuccess) return TV_ERR_HIP;
  }
  return TV_OK;
}

}  // namespace tv
