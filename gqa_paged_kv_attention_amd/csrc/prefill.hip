// Mixed chunked-prefill + decode batch over the paged cache, bf16: a
// scheduling pass and one fused kernel.
//
// The mixed batch of "[Kernel] [V1] Further optimizations to ROCm (Triton)
// Backend to better handle GQA" (vLLM PR #14431, review thread on
// chunked_prefill_paged_decode) holds sequences with more than one new token
// (prefill chunks: each new token attends causally to the cached prefix and to
// the chunk's earlier tokens, bottom-right aligned) and sequences with one new
// token (decodes), which the thread runs as a prefill kernel plus a decode
// kernel launched alongside it.  Here both kinds of work are units of one
// launch, ordered by a scheduling pass (below).
//
// The prefill role (GQA row packing, LDS-shared K/V tiles, matrix-core
// products) is in prefill_core.h.
#include "prefill_core.h"

namespace gqa {

namespace {

// ---------------------------------------------------------------------------
// Scheduling pass.  The mixed batch splits into work units, each run by one
// work-group per kv head: a prefill row tile of a sequence with q_len > 1, or
// a decode partition of a sequence with q_len = 1.  Their costs differ by
// orders of magnitude (a row tile near the end of a long chunk reads the whole
// prefix; most decodes read a few pages), and work-groups are dispatched in
// index order, so sequences are listed by decreasing cost of their costliest
// unit (longest processing time first): the long units start first and the
// short ones fill in behind them.  Prefill and decode units form two such
// lists, merged in proportion to their lengths, so that the HBM-bound decodes
// run beside the matrix-bound prefill tiles all through the launch rather
// than after them.  A sequence's units stay contiguous, heaviest
// first: its row tiles then run at the same time and stream the same K/V
// pages, which they mostly find in L2 instead of each fetching the prefix from
// HBM (work-group i goes to XCD i mod 8, so with Hkv a multiple of 8 all work-
// groups of one kv head share an XCD and its L2).  Cost,
// in tile steps of a work-group: a prefill row tile takes one step per 32-key
// tile up to its last row's causal limit; a decode partition's tiles are
// shared by the waves.  One work-group of 1024 threads counts the units per
// cost bucket and list in LDS, scans, and reserves a range per sequence (the
// order of sequences within a bucket is arbitrary; each unit's result does not
// depend on it).
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kCostBuckets = 2048;

__device__ __forceinline__ int unit_cost_bucket(int c) { return min(c, kCostBuckets - 1); }

// Units of sequence b and the cost of its costliest unit, without walking
// them: the last row tile reaches furthest, and the first decode partition
// holds the extra tile of an uneven split.  Both are 0 for a sequence that
// produces no work.
struct SeqInfo {
  int q0, q1, seq_len;
};

__device__ __forceinline__ bool seq_summary(const ScheduleArgs& a, int b, int* units, int* cost, SeqInfo* info) {
  *units = 0;
  *cost = 0;
  const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
  const int sl = a.seq_lens[b];
  *info = SeqInfo{q0, q1, sl};
  const int q_len = q1 - q0;
  if (q1 > a.num_tokens || q0 < 0 || q_len <= 0 || q_len > a.max_query_len) return false;
  const int L = clamp_len(sl, a.max_blocks_per_seq, a.block_size);
  if (q_len == 1) {
    const int Lp = min(L, a.max_partitions * a.partition_size);
    const int nparts = max(1, (Lp + a.partition_size - 1) / a.partition_size);
    const int tiles_all = (Lp + kTile - 1) / kTile;
    const int first = tiles_all / nparts + (tiles_all % nparts ? 1 : 0);
    *units = nparts;
    *cost = first;
    return true;
  }
  const int prior = L - q_len;
  if (a.causal && prior < 0) return false;
  *units = (q_len * a.group + a.rows_per_group - 1) / a.rows_per_group;
  // tiles up to the last row's last visible key (all L keys without the mask)
  *cost = (a.causal ? prior + q_len - 1 : max(L - 1, 0)) / kTile + 1;
  return false;
}

// Exclusive prefix sum of one value per thread over the work-group (wave
// scans, then a scan of the 16 wave totals); *total gets the sum of all.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < kSchedThreads / 64 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < kSchedThreads / 64; off <<= 1) {
      const int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < kSchedThreads / 64) wsum[lane] = t;
  }
  __syncthreads();
  *total = wsum[kSchedThreads / 64 - 1];
  const int base = w ? wsum[w - 1] : 0;
  __syncthreads();
  return base + x - v;
}

// Positions in the merged list of elements r, r + 1, ... of one list when the
// prefill and decode lists (n_self and n_other elements) are interleaved in
// proportion: element i of the prefill list sits at key (2i + 1) n_decode,
// element j of the decode list at (2j + 1) n_prefill, prefill first on ties.
// The count of other-list elements before element r is a quotient of
// num(r) = (2r + 1) n_other - n_self by den = 2 n_self (ceiling for prefill,
// floor + 1 for decode, clamped to [0, n_other]); it is kept as an exact
// quotient and remainder and stepped by 2 n_other per element.
struct MergeCursor {
  long long q;                  // floor(num / den)
  int rem, den, step_q, step_r, n_other, r;
  bool decode;
  __device__ __forceinline__ MergeCursor(int r0, int n_self, int n_oth, bool is_decode) {
    den = 2 * n_self;
    n_other = n_oth;
    r = r0;
    decode = is_decode;
    const long long num = (2LL * r0 + 1) * n_oth - n_self;
    // floor division of a possibly negative 64-bit value by a positive int
    q = num >= 0 ? num / den : -((-num + den - 1) / den);
    rem = (int)(num - q * den);
    step_q = (2 * n_oth) / den;
    step_r = (2 * n_oth) % den;
  }
  __device__ __forceinline__ int position() const {
    long long before = decode ? (q >= 0 ? q + 1 : 0) : (q + (rem > 0 ? 1 : 0));
    before = before < 0 ? 0 : (before > n_other ? n_other : before);
    return r + (int)before;
  }
  __device__ __forceinline__ void next() {
    ++r;
    q += step_q;
    rem += step_r;
    if (rem >= den) {
      rem -= den;
      ++q;
    }
  }
};

// Position in the merged list of element r of one list, as MergeCursor gives
// it, from the closed form: the quotient (2r + 1) n_other - n_self over
// 2 n_self, in double precision.  It is exact: |numerator| < 2^41 and the
// quotient < 2^21, so the rounding error (< 2^-32) cannot cross the distance
// 1 / (2 n_self) >= 2^-21 to the next integer, and exact quotients are exact.
__device__ __forceinline__ int merged_position(int r, int n_self, int n_other, bool decode) {
  const double num = (2.0 * r + 1.0) * n_other - n_self;
  const double qt = num / (2.0 * n_self);
  long long before = decode ? (long long)floor(qt) + 1 : (long long)ceil(qt);
  before = before < 0 ? 0 : (before > n_other ? n_other : before);
  return r + (int)before;
}

// Sizes of the two lists of the merged order.  Prefill row tiles are one unit
// each.  Decode partitions are listed costliest first: the n_long partitions of
// more than kWaveDecodeMaxTiles tiles are one (whole work-group) unit each; the
// rest are packed four to a unit, one per wave, so that neighbours in a pack
// have similar lengths.
struct ListSizes {
  int n_pf, n_dec, n_long, n_du;
};

// block_tables[b][min(j, pages - 1)] for j = 0..7: the pages of a prefill
// unit's first two 64-key tiles.
__device__ __forceinline__ void first_pages(const ScheduleArgs& a, int b, int seq_len, int e[8]) {
  const int L = clamp_len(seq_len, a.max_blocks_per_seq, a.block_size);
  const int last = max((L + a.block_size - 1) / a.block_size - 1, 0);
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = bt[min(j, last)];
}

__device__ __forceinline__ void write_prefill_unit(const ScheduleArgs& a, int pos, int b, int rt, const SeqInfo& in,
                                                   const int e[8]) {
  if (pos >= a.unit_capacity) return;
  a.units[pos].s[0] = make_int4(b, rt, in.q0, in.q1);
  a.units[pos].s[1] = make_int4(in.seq_len, 0, 0, 0);
  a.units[pos].s[2] = make_int4(e[0], e[1], e[2], e[3]);
  a.units[pos].s[3] = make_int4(e[4], e[5], e[6], e[7]);
}

// Decode partition k of sequence b, element r of the decode list.
__device__ __forceinline__ void write_decode_element(const ScheduleArgs& a, const ListSizes& z, int r, int b, int k,
                                                     const SeqInfo& in) {
  const int4 e = make_int4(b, -1 - k, in.q0, in.seq_len);
  if (r < z.n_long) {
    const int pos = merged_position(r, z.n_du, z.n_pf, true);
    if (pos >= a.unit_capacity) return;
    a.units[pos].s[0] = e;
    a.units[pos].s[1] = make_int4(kUnitWholeGroup, 0, 0, 0);
    return;
  }
  const int sr = r - z.n_long, pack = sr / 4, w = sr % 4;
  const int pos = merged_position(z.n_long + pack, z.n_du, z.n_pf, true);
  if (pos >= a.unit_capacity) return;
  a.units[pos].s[w] = e;
  if (w == 0)
    for (int j = min(4, z.n_dec - z.n_long - 4 * pack); j < 4; ++j)
      a.units[pos].s[j] = make_int4(kUnitEmpty, 0, 0, 0);
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(ScheduleArgs a) {
  __shared__ int hist[2][kCostBuckets];      // [prefill, decode][cost bucket]
  __shared__ int wsum[kSchedThreads / 64];
  // one sequence per thread (num_seqs <= kSchedThreads): flat start of its
  // units, start in its list, unit count (negative: decode list), query range and length
  __shared__ int s_flat[kSchedThreads], s_r0[kSchedThreads], s_nu[kSchedThreads];
  __shared__ int s_info[kSchedThreads][3];
  __shared__ int s_pages[kSchedThreads][8];   // first_pages() of a prefill sequence
  for (int i = threadIdx.x; i < 2 * kCostBuckets; i += kSchedThreads) hist[i / kCostBuckets][i % kCostBuckets] = 0;
  __syncthreads();
  // the summary of this thread's first sequence is kept for the second pass
  int nu0 = 0, cmax0 = 0;
  bool dec0 = false;
  SeqInfo info0{0, 0, 0};
  int pages0[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int b = threadIdx.x; b < a.num_seqs; b += kSchedThreads) {
    int nu, cmax;
    SeqInfo info;
    const bool dec = seq_summary(a, b, &nu, &cmax, &info);
    if (b == threadIdx.x) {
      nu0 = nu;
      cmax0 = cmax;
      dec0 = dec;
      info0 = info;
      // loaded now, so that the loads overlap the scans below
      if (nu && !dec) first_pages(a, b, info.seq_len, pages0);
    }
    if (nu) atomicAdd(&hist[dec][unit_cost_bucket(cmax)], nu);
  }
  __syncthreads();
  // exclusive scans in decreasing cost: start[c] = units of that list costlier than c
  constexpr int PER = kCostBuckets / kSchedThreads;
  const int top = kCostBuckets - 1 - PER * threadIdx.x;       // this thread's buckets: top, top-1, ...
  int n_list[2];
#pragma unroll
  for (int l = 0; l < 2; ++l) {
    int local[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      local[i] = hist[l][top - i];
      sum += local[i];
    }
    int run = block_exclusive_scan(sum, &n_list[l], wsum);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      hist[l][top - i] = run;
      run += local[i];
    }
  }
  __syncthreads();
  // decode partitions costlier than kWaveDecodeMaxTiles tiles: the start of its bucket
  ListSizes z;
  z.n_pf = n_list[0];
  z.n_dec = n_list[1];
  z.n_long = hist[1][unit_cost_bucket(kWaveDecodeMaxTiles)];
  z.n_du = z.n_long + (z.n_dec - z.n_long + 3) / 4;
  __syncthreads();
  if (a.num_seqs <= kSchedThreads) {
    // One sequence per thread: each reserves its range, then all threads
    // write the units together (a long chunk's units would otherwise be
    // written one after another by its thread, which sets the kernel's end).
    const int b = threadIdx.x;
    int nu = 0, r0 = 0;
    if (b < a.num_seqs && nu0) {
      nu = nu0;
      r0 = atomicAdd(&hist[dec0][unit_cost_bucket(cmax0)], nu0);
    }
    int total;
    const int flat = block_exclusive_scan(nu, &total, wsum);
    s_flat[b] = flat;
    s_r0[b] = r0;
    s_nu[b] = dec0 ? -nu : nu;
    s_info[b][0] = info0.q0;
    s_info[b][1] = info0.q1;
    s_info[b][2] = info0.seq_len;
#pragma unroll
    for (int j = 0; j < 8; ++j) s_pages[b][j] = pages0[j];
    __syncthreads();
    for (int f = threadIdx.x; f < total; f += kSchedThreads) {
      // owner: the last sequence whose flat start is <= f (ranges are in
      // sequence order; an empty sequence shares its successor's start, so
      // the last such sequence is never empty)
      int lo = 0, hi = kSchedThreads;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_flat[mid] <= f) lo = mid; else hi = mid;
      }
      const bool dec = s_nu[lo] < 0;
      const int n = dec ? -s_nu[lo] : s_nu[lo];
      const int k = f - s_flat[lo];
      const SeqInfo in{s_info[lo][0], s_info[lo][1], s_info[lo][2]};
      if (dec)
        write_decode_element(a, z, s_r0[lo] + k, lo, k, in);
      else
        write_prefill_unit(a, merged_position(s_r0[lo] + k, z.n_pf, z.n_du, false), lo, n - 1 - k, in, s_pages[lo]);
    }
  } else {
    for (int b = threadIdx.x; b < a.num_seqs; b += kSchedThreads) {
      int nu = nu0, cmax = cmax0;
      bool dec = dec0;
      SeqInfo info = info0;
      if (b != threadIdx.x) dec = seq_summary(a, b, &nu, &cmax, &info);
      if (!nu) continue;
      // a contiguous range of its list; units heaviest first (the last row tile
      // reaches furthest; decode partitions are in order)
      const int r0 = atomicAdd(&hist[dec][unit_cost_bucket(cmax)], nu);
      if (dec) {
        for (int k = 0; k < nu; ++k) write_decode_element(a, z, r0 + k, b, k, info);
      } else {
        int e[8];
        first_pages(a, b, info.seq_len, e);
        MergeCursor cur(r0, z.n_pf, z.n_du, false);
        for (int k = 0; k < nu; ++k, cur.next()) write_prefill_unit(a, cur.position(), b, nu - 1 - k, info, e);
      }
    }
  }
  if (threadIdx.x == 0) *a.unit_count = min(z.n_pf + z.n_du, a.unit_capacity);
}

// ---------------------------------------------------------------------------
// Mixed batch: work-group i runs unit i / Hkv of the scheduled list for kv
// head i % Hkv, as a prefill row tile (K/V tiles shared through LDS) or as a
// decode partition (per-wave tile pipeline, waves merged through LDS).  The
// decode units ride along the prefill ones in one launch: HBM-bound decodes
// and matrix-bound prefill tiles then share the device instead of running one
// after the other.
// ---------------------------------------------------------------------------
template <int D, int NT, int BS, class OutT, int W>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1)))
void mixed_kernel(MixedArgs a) {
  typedef PrefillLds<D, kLdsNTW, W> S;
  __shared__ __attribute__((aligned(16))) char lds[MixedLds<D, NT, W>::kBytes];
  const int Hkv = a.prefill.num_kv_heads;
  const int slot = blockIdx.x / Hkv, kv = blockIdx.x % Hkv;
  // the record is read together with the count (slot < the list's capacity)
  const int count = *a.unit_count;
  const int4 u = a.units[slot].s[0];
  const int4 u1 = a.units[slot].s[1];
  if (slot >= count) return;
  if (u.y >= 0) {
    uint16_t* sK = reinterpret_cast<uint16_t*>(lds);
    const int4 p0 = a.units[slot].s[2], p1 = a.units[slot].s[3];
    const int first_pages[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    prefill_unit<D, kLdsNTW, BS, OutT, W>(a.prefill, u.x, u.y, u.z, u.w, u1.x, kv, sK, sK + 2 * S::KBUF, 0,
                                          UnitOut(), first_pages);
  } else if (u1.x == kUnitWholeGroup) {
    decode_partition_at<TileBF16<D, BS>, D, NT, OutT, W>(a.decode, -1 - u.y, kv, u.x, u.z, u.w,
                                                         reinterpret_cast<float*>(lds));
  } else {
    // one short decode partition per wave, four to a record (the branch is
    // uniform per wave; with 8 waves the last four have none)
    const int w = wave_id();
    if (w < kPackSlots) {
      const int4 e = a.units[slot].s[w];
      if (e.x >= 0) decode_wave_partition<TileBF16<D, BS>, D, NT, OutT>(a.decode, -1 - e.y, kv, e.x, e.z, e.w);
    }
  }
}

template <int D, int BS, class OutT>
hipError_t mixed_dispatch(const MixedArgs& a, int groups, int waves, hipStream_t s) {
  if (a.prefill.group > 16)
    return launch_kernel(mixed_kernel<D, 2, BS, OutT, kWaves>, dim3(groups), dim3(kThreads), 0, s, a);
  if (waves == 2 * kWaves)
    return launch_kernel(mixed_kernel<D, 1, BS, OutT, 2 * kWaves>, dim3(groups), dim3(2 * kThreads), 0, s, a);
  return launch_kernel(mixed_kernel<D, 1, BS, OutT, kWaves>, dim3(groups), dim3(kThreads), 0, s, a);
}

}  // namespace

int prefill_lds_rows_per_group(int waves) {
  return waves == 2 * kWaves ? PrefillLds<128, kLdsNTW, 2 * kWaves>::kRowsPerGroup
                             : PrefillLds<128, kLdsNTW>::kRowsPerGroup;
}

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t stream) {
  return launch_kernel(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a);
}

hipError_t launch_mixed(const MixedArgs& a, int head_dim, int block_size, bool out_f32, int grid_groups, int waves,
                        hipStream_t stream) {
  // the scheduling pass cut the prefill rows for this wave count: only the
  // launches that exist for it (8 waves: G <= 16)
  if (waves != kWaves && (waves != 2 * kWaves || a.prefill.group > 16)) return hipErrorInvalidValue;
  return with_block_size(block_size, [&](auto bs) {
    constexpr int BS = decltype(bs)::value;
    if (head_dim == 64)
      return out_f32 ? mixed_dispatch<64, BS, float>(a, grid_groups, waves, stream)
                     : mixed_dispatch<64, BS, uint16_t>(a, grid_groups, waves, stream);
    return out_f32 ? mixed_dispatch<128, BS, float>(a, grid_groups, waves, stream)
                   : mixed_dispatch<128, BS, uint16_t>(a, grid_groups, waves, stream);
  });
}

}  // namespace gqa
