// Random calls of the host entry points of include/sink_attn.h (the tile
// schedule calls of the packed, padded and paged families), valid and
// invalid alike, for the host sanitizer test. Every array the library may
// read is allocated at exactly the size the header states, so an
// out-of-bounds read, an overflow or other undefined behaviour in the
// argument checks or the table builder shows up under AddressSanitizer /
// UndefinedBehaviorSanitizer. Prints one line per call:
//   case <i> <family> <status> <words> <fwd bytes> <bwd bytes> <FNV-1a of the table>
// so that the same program linked against libsinkattn.so can be compared
// line by line. usage: fuzz_metadata SEED COUNT
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "sink_attn.h"

namespace {

uint64_t g_state = 1;

// splitmix64: input generation only
uint64_t next_u64() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int32_t pick(int32_t lo, int32_t hi) {  // uniform in [lo, hi]
  return lo + static_cast<int32_t>(next_u64() % static_cast<uint64_t>(hi - lo + 1));
}

bool chance(int percent) { return pick(0, 99) < percent; }

int32_t odd_value() {
  static const int32_t v[] = {-2, -1, 0, 1, 3, 100, 255, 4097, 65535, 65536, INT_MAX, INT_MIN};
  return v[pick(0, static_cast<int32_t>(sizeof(v) / sizeof(v[0])) - 1)];
}

uint64_t fnv(uint64_t h, const void* p, size_t n) {
  const unsigned char* b = static_cast<const unsigned char*>(p);
  for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 0x100000001B3ull;
  return h;
}

struct Result {
  int status = 0;
  int64_t words = 0, fws = 0, bws = 0;
  uint64_t hash = 0xCBF29CE484222325ull;
};

// size query, then the table at exactly that size, then one word short
template <typename Call>
Result run(Call call) {
  Result r;
  int64_t words = -7, fws = -7, bws = -7;
  r.status = call(nullptr, 0, &words, &fws, &bws);
  if (r.status != SINK_ATTN_OK) return r;
  if (words <= 0) {
    std::printf("bad size %lld\n", static_cast<long long>(words));
    std::exit(2);
  }
  std::vector<int32_t> meta(static_cast<size_t>(words));
  int64_t words2 = 0, fws2 = 0, bws2 = 0;
  const int st = call(meta.data(), words, &words2, &fws2, &bws2);
  if (st != SINK_ATTN_OK || words2 != words || fws2 != fws || bws2 != bws) {
    std::printf("second call differs: %d\n", st);
    std::exit(2);
  }
  std::vector<int32_t> shorter(static_cast<size_t>(words - 1));   // the header alone is 56 words
  if (call(shorter.data(), words - 1, &words2, &fws2, &bws2) != SINK_ATTN_E_BUFFER_TOO_SMALL) {
    std::printf("short buffer accepted\n");
    std::exit(2);
  }
  r.words = words;
  r.fws = fws;
  r.bws = bws;
  r.hash = fnv(r.hash, meta.data(), meta.size() * sizeof(int32_t));
  return r;
}

sink_attn_problem random_problem(int batch) {
  sink_attn_problem p = {};
  p.batch = batch;
  static const int32_t hk_choice[] = {1, 2, 8};
  p.num_heads_k = hk_choice[pick(0, 2)];
  p.num_heads_q = p.num_heads_k * pick(1, 8);
  static const int32_t d_choice[] = {64, 128, 256};
  p.head_dim = d_choice[pick(0, 2)];
  p.causal = pick(0, 1);
  p.win_left = chance(50) ? -1 : pick(0, 3000);
  p.win_right = p.causal ? (chance(50) ? -1 : 0) : (chance(50) ? -1 : pick(0, 3000));
  p.dtype = pick(0, 2);
  return p;
}

// one field of the problem replaced by an odd value
void corrupt(sink_attn_problem& p) {
  int32_t* fields[] = {&p.batch, &p.num_heads_q, &p.num_heads_k, &p.head_dim, &p.total_q,
                       &p.total_k, &p.max_seqlen_q, &p.max_seqlen_k, &p.causal, &p.win_left,
                       &p.win_right, &p.dtype, &p.layout_q, &p.layout_out, &p.seq_q, &p.seq_k};
  *fields[pick(0, 15)] = odd_value();
}

std::vector<int32_t> lengths(int n, int32_t hi) {
  std::vector<int32_t> v(static_cast<size_t>(n));
  for (auto& x : v) x = chance(10) ? 0 : pick(1, hi);
  return v;
}

Result packed_case() {
  const int batch = pick(1, 24);
  sink_attn_problem p = random_problem(batch);
  const std::vector<int32_t> lq = lengths(batch, chance(30) ? 16 : 3000);
  const std::vector<int32_t> lk = lengths(batch, 5000);
  std::vector<int32_t> cq(static_cast<size_t>(batch) + 1, 0), ck(static_cast<size_t>(batch) + 1, 0);
  for (int b = 0; b < batch; ++b) {
    cq[b + 1] = cq[b] + lq[b];
    ck[b + 1] = ck[b] + lk[b];
    p.max_seqlen_q = lq[b] > p.max_seqlen_q ? lq[b] : p.max_seqlen_q;
    p.max_seqlen_k = lk[b] > p.max_seqlen_k ? lk[b] : p.max_seqlen_k;
  }
  p.total_q = cq[batch];
  p.total_k = ck[batch];
  if (chance(20)) {                              // cu_seqlens out of order or off by one
    const int b = pick(0, batch);
    (chance(50) ? cq : ck)[b] += pick(-3, 3);
  }
  if (chance(20)) corrupt(p);
  // the arrays hold batch + 1 entries of the batch drawn above, whatever the field says
  if (p.batch != batch && p.batch > 0 && p.batch < 65536) p.batch = batch;
  return run([&](int32_t* m, int64_t cap, int64_t* w, int64_t* f, int64_t* b) {
    return static_cast<int>(sink_attn_metadata(&p, cq.data(), ck.data(), m, cap, w, f, b));
  });
}

Result padded_case() {
  const int batch = pick(1, 16);
  sink_attn_problem p = random_problem(batch);
  p.layout_q = pick(1, 2);
  p.layout_out = (p.layout_q == SINK_ATTN_BNSD && chance(30)) ? SINK_ATTN_BSND : p.layout_q;
  p.seq_q = pick(1, 2000);
  p.seq_k = pick(1, 3000);
  p.total_q = batch * p.seq_q;
  p.total_k = batch * p.seq_k;
  std::vector<int32_t> uq = lengths(batch, p.seq_q), uk = lengths(batch, p.seq_k);
  const bool use_q = chance(60), use_k = chance(60);
  p.max_seqlen_q = p.max_seqlen_k = 0;
  for (int b = 0; b < batch; ++b) {
    const int32_t a = use_q ? uq[b] : p.seq_q, c = use_k ? uk[b] : p.seq_k;
    p.max_seqlen_q = a > p.max_seqlen_q ? a : p.max_seqlen_q;
    p.max_seqlen_k = c > p.max_seqlen_k ? c : p.max_seqlen_k;
  }
  if (chance(15)) uq[static_cast<size_t>(pick(0, batch - 1))] = odd_value();
  if (chance(20)) corrupt(p);
  if (p.batch != batch && p.batch > 0 && p.batch < 65536) p.batch = batch;
  return run([&](int32_t* m, int64_t cap, int64_t* w, int64_t* f, int64_t* b) {
    return static_cast<int>(sink_attn_metadata_padded(&p, use_q ? uq.data() : nullptr,
                                                      use_k ? uk.data() : nullptr, m, cap, w,
                                                      f, b));
  });
}

Result paged_case() {
  const int batch = pick(1, 16);
  sink_attn_problem p = random_problem(batch);
  sink_attn_paged_kv kv = {};
  static const int32_t bs_choice[] = {16, 32, 64, 256, 1024};
  kv.block_size = bs_choice[pick(0, 4)];
  kv.layout = pick(0, 1);
  const std::vector<int32_t> lq = lengths(batch, chance(60) ? 16 : 700);
  const std::vector<int32_t> used = lengths(batch, 9000);
  std::vector<int32_t> cq(static_cast<size_t>(batch) + 1, 0);
  int32_t pages_max = 1;
  p.max_seqlen_q = p.max_seqlen_k = p.total_k = 0;
  for (int b = 0; b < batch; ++b) {
    cq[b + 1] = cq[b] + lq[b];
    p.max_seqlen_q = lq[b] > p.max_seqlen_q ? lq[b] : p.max_seqlen_q;
    p.max_seqlen_k = used[b] > p.max_seqlen_k ? used[b] : p.max_seqlen_k;
    p.total_k += used[b];
    const int32_t pages = (used[b] + kv.block_size - 1) / kv.block_size;
    pages_max = pages > pages_max ? pages : pages_max;
  }
  p.total_q = cq[batch];
  kv.max_blocks_per_seq = pages_max + pick(0, 2) - (chance(10) ? 1 : 0);
  kv.num_blocks = pick(1, 4000);
  if (kv.max_blocks_per_seq < 1) kv.max_blocks_per_seq = 1;
  std::vector<int32_t> table(static_cast<size_t>(batch) * kv.max_blocks_per_seq);
  for (auto& t : table) t = pick(0, kv.num_blocks - 1);
  if (chance(15)) table[static_cast<size_t>(pick(0, static_cast<int32_t>(table.size()) - 1))] = odd_value();
  if (chance(15)) kv.block_size = odd_value();
  if (chance(20)) corrupt(p);
  if (p.batch != batch && p.batch > 0 && p.batch < 65536) p.batch = batch;
  return run([&](int32_t* m, int64_t cap, int64_t* w, int64_t* f, int64_t* b) {
    *b = 0;
    return static_cast<int>(sink_attn_metadata_paged(&p, &kv, cq.data(), used.data(),
                                                     table.data(), m, cap, w, f));
  });
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) return 1;
  g_state = std::strtoull(argv[1], nullptr, 10);
  const int count = std::atoi(argv[2]);
  int ok = 0;
  for (int i = 0; i < count; ++i) {
    const int family = pick(0, 2);
    const Result r = family == 0 ? packed_case() : family == 1 ? padded_case() : paged_case();
    ok += r.status == SINK_ATTN_OK;
    std::printf("case %d %d %d %lld %lld %lld %016llx\n", i, family, r.status,
                static_cast<long long>(r.words), static_cast<long long>(r.fws),
                static_cast<long long>(r.bws), static_cast<unsigned long long>(r.hash));
  }
  std::printf("ok %d of %d\n", ok, count);
  return 0;
}
