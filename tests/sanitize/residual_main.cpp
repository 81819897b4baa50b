// Test driver: runs the host residual routine of the library (residual_host.cpp, compiled into this
// executable with the host compiler) on inputs written by the test to a directory, and writes its
// output there.  Built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py; it links nothing else of the library (no HIP).
//
//   residual_main DIR   reads DIR/params.txt ("fmt n_experts d I T E k threads has_mask has_slots")
//                       and the raw arrays DIR/{w13,w2,s13,s2,x,ids,w,mask,slots}.bin;
//                       writes DIR/out.bin (fp32 [T][d]) and prints the pair count.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <string>
#include <vector>

namespace ftk {
int residual_host(int fmt, int n_experts, int d, int I, const uint8_t* w13, const uint8_t* w2, const uint8_t* s13,
                  const uint8_t* s2, const uint16_t* x, const int32_t* ids, const float* w, const uint32_t* mask,
                  const int32_t* slot_of_expert, int T, int E, int k, float* out, int threads);
}

static std::vector<uint8_t> read_file(const std::string& path, bool required) {
  std::vector<uint8_t> buf;
  FILE* f = fopen(path.c_str(), "rb");
  if (!f) {
    if (required) {
      fprintf(stderr, "cannot open %s\n", path.c_str());
      exit(2);
    }
    return buf;
  }
  fseek(f, 0, SEEK_END);
  const long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  buf.resize((size_t)n);
  if (n > 0 && fread(buf.data(), 1, (size_t)n, f) != (size_t)n) exit(2);
  fclose(f);
  return buf;
}

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  const std::string dir = argv[1];
  int fmt, n_experts, d, I, T, E, k, threads, has_mask, has_slots;
  FILE* p = fopen((dir + "/params.txt").c_str(), "r");
  if (!p || fscanf(p, "%d %d %d %d %d %d %d %d %d %d", &fmt, &n_experts, &d, &I, &T, &E, &k, &threads, &has_mask,
                   &has_slots) != 10)
    return 2;
  fclose(p);
  // exact-size heap copies, so an access past any array is reported
  auto w13 = read_file(dir + "/w13.bin", true), w2 = read_file(dir + "/w2.bin", true);
  auto s13 = read_file(dir + "/s13.bin", false), s2 = read_file(dir + "/s2.bin", false);
  auto x = read_file(dir + "/x.bin", true), ids = read_file(dir + "/ids.bin", true), w = read_file(dir + "/w.bin", true);
  auto mask = read_file(dir + "/mask.bin", false), slots = read_file(dir + "/slots.bin", false);
  std::vector<float> out((size_t)T * d);
  const int n = ftk::residual_host(fmt, n_experts, d, I, w13.data(), w2.data(), s13.empty() ? nullptr : s13.data(),
                                   s2.empty() ? nullptr : s2.data(), (const uint16_t*)x.data(),
                                   (const int32_t*)ids.data(), (const float*)w.data(),
                                   has_mask ? (const uint32_t*)mask.data() : nullptr,
                                   has_slots ? (const int32_t*)slots.data() : nullptr, T, E, k, out.data(), threads);
  FILE* o = fopen((dir + "/out.bin").c_str(), "wb");
  if (!o || fwrite(out.data(), sizeof(float), out.size(), o) != out.size()) return 2;
  fclose(o);
  printf("%d\n", n);
  return 0;
}
