// Driver of the host-built combine kernels (CPU tests only): moe_combine_release's list path
// (the link kernel, the merge kernel, then the release compaction done plainly) over the calls
// read from a directory; fp32 rows and fp32 outputs.  Usage: combine_host <dir>.
#include "shim.hpp"
#include <cstdio>
#include <cstdlib>
#include <string>

#include "combine_link.hpp"  // the link step the link kernel runs (namespace moe)

namespace moe {
#include "combine_kernels.inc"  // the kernels, cut from combine.hip by the test
}
using namespace moe;

template <typename T>
static T* rd(const std::string& dir, const std::string& name, size_t n) {
  T* p = (T*)std::malloc(n ? n * sizeof(T) : 1);
  if (n) {
    FILE* f = std::fopen((dir + "/" + name).c_str(), "rb");
    if (!f || std::fread(p, sizeof(T), n, f) != n) { std::fprintf(stderr, "cannot read %s\n", name.c_str()); std::exit(2); }
    std::fclose(f);
  }
  return p;
}

template <typename T>
static void wr(const std::string& dir, const std::string& name, const T* p, size_t n) {
  FILE* f = std::fopen((dir + "/" + name).c_str(), "wb");
  std::fwrite(p, sizeof(T), n, f);
  std::fclose(f);
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const std::string dir = argv[1];
  int T_cap, H, K, calls;
  {
    FILE* f = std::fopen((dir + "/meta.txt").c_str(), "r");
    if (!f || std::fscanf(f, "%d %d %d %d", &T_cap, &H, &K, &calls) != 4) return 2;
    std::fclose(f);
  }
  float* acc = (float*)std::calloc((size_t)T_cap * H, 4);
  float* out = (float*)std::calloc((size_t)T_cap * H, 4);
  uint32_t* mask = (uint32_t*)std::calloc(T_cap, 4);
  uint32_t* tgen = (uint32_t*)std::calloc(T_cap, 4);
  uint8_t* rflag = (uint8_t*)std::calloc(T_cap, 1);
  int* head = (int*)std::malloc((size_t)T_cap * 4);
  for (int t = 0; t < T_cap; ++t) head[t] = -1;
  uint32_t err = 0;
  for (int c = 0; c < calls; ++c) {
    const std::string p = "c" + std::to_string(c) + "_";
    int m, n_rows;
    {
      FILE* f = std::fopen((dir + "/" + p + "meta.txt").c_str(), "r");
      if (!f || std::fscanf(f, "%d %d", &m, &n_rows) != 2) return 2;
      std::fclose(f);
    }
    float* rows = rd<float>(dir, p + "rows", (size_t)n_rows * H);
    int* ri = rd<int>(dir, p + "row_idx", m);
    int* tk = rd<int>(dir, p + "tok", m);
    int* ks = rd<int>(dir, p + "kslot", m);
    float* w = rd<float>(dir, p + "w", m);
    uint32_t* g = rd<uint32_t>(dir, p + "gen", m);
    // the list path's workspace: next[m], then the tokens' masks before the call
    int32_t* ws = (int32_t*)std::malloc((size_t)m * 8 + 16);
    LinkJob lj;
    lj.m = m;
    lj.K = K;
    lj.T_cap = T_cap;
    lj.n_rows = n_rows;
    lj.tok = tk;
    lj.kslot = ks;
    lj.gen = g;
    lj.tgen = tgen;
    lj.mask = mask;
    lj.head = head;
    lj.next = ws;
    lj.mpre = (uint32_t*)ws + m;
    lj.err = &err;
    run_grid((m + 255) / 256, 256, [&] { combine_link_kernel(lj, ri); });
    auto merge = [&](auto vc) {
      constexpr int V = decltype(vc)::value;
      run_grid(m, kMergeThreads, [&] {
        combine_merge_kernel<float, float, V>(K, H, rows, H, ri, tk, ks, w, acc, mask, tgen, rflag, head, ws,
                                              (const uint32_t*)ws + m, out, H, &err);
      });
    };
    const int vpt = (H / 8 + kMergeThreads - 1) / kMergeThreads;
    if (m > 0) {
      if (vpt <= 1) merge(std::integral_constant<int, 1>{});
      else if (vpt <= 2) merge(std::integral_constant<int, 2>{});
      else if (vpt <= kMergeVec) merge(std::integral_constant<int, kMergeVec>{});
      else merge(std::integral_constant<int, 0>{});
    }
    std::vector<int> rel;
    for (int t = 0; t < T_cap; ++t)
      if (rflag[t]) { rel.push_back(t); rflag[t] = 0; }
    wr(dir, p + "rel.bin", rel.data(), rel.size());
    for (int t = 0; t < T_cap; ++t)
      if (head[t] != -1) { std::fprintf(stderr, "head[%d] not reset\n", t); return 3; }
    std::free(rows); std::free(ri); std::free(tk); std::free(ks); std::free(w); std::free(g); std::free(ws);
  }
  wr(dir, "out.bin", out, (size_t)T_cap * H);
  wr(dir, "mask.bin", mask, T_cap);
  wr(dir, "tgen.bin", tgen, T_cap);
  wr(dir, "err.bin", &err, 1);
  return 0;
}
