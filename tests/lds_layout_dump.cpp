// Prints the LDS fill and fragment-read offsets that the kernels compute
// (attention_flash_sdpa_amd/csrc/lds_layout.h, built here for the host) as one
// JSON object, for the CPU model of the LDS banks in test_lds_banks.py.
#include <cstdio>

#include "lds_layout.h"

using namespace sdpa;

namespace {

bool first_key = true;

void key(const char* name) {
  std::printf("%s\"%s\": ", first_key ? "" : ",\n", name);
  first_key = false;
}

template <class F>
void list(int n, F f) {
  std::printf("[");
  for (int i = 0; i < n; ++i) {
    if (i) std::printf(",");
    f(i);
  }
  std::printf("]");
}

void lanes(unsigned (*f)(unsigned, unsigned, unsigned), unsigned a, unsigned b) {
  list(64, [&](int l) { std::printf("%u", f((unsigned)l, a, b)); });
}

template <int SLOTS> unsigned k16(unsigned l, unsigned s, unsigned) { return prefill_k_read<SLOTS>(l, s); }
template <int SLOTS> unsigned vt16(unsigned l, unsigned hf, unsigned t) { return prefill_vt_read<SLOTS>(l, hf, t); }
unsigned ka8(unsigned l, unsigned s, unsigned c) { return fp8_ka_read(l, s, c); }
unsigned kb8(unsigned l, unsigned c, unsigned) { return fp8_kb_read(l, c); }
unsigned vt8(unsigned l, unsigned t, unsigned) { return fp8_vt_read(l, t); }
template <int SLOTS> unsigned dk(unsigned l, unsigned s, unsigned) { return decode_k_read<SLOTS>(l, s); }
template <int SLOTS> unsigned dvt(unsigned l, unsigned hf, unsigned t) { return decode_vt_read<SLOTS>(l, hf, t); }

template <class F>
void fill(const char* name, int slots, F f) {
  key(name);
  list(slots, [&](int s) { std::printf("%u", f((unsigned)s)); });
}

}  // namespace

int main() {
  std::printf("{\n");
  // fills of one block: 64 keys (prefill) or 32 keys (decode)
  fill("fill_prefill16", 64 * 16, [](unsigned s) { return fill_chunk_prefill<16>(s); });
  fill("fill_prefill8", 64 * 8, [](unsigned s) { return fill_chunk_prefill<8>(s); });
  fill("fill_quarter", 64 * 4, [](unsigned s) { return fill_chunk_quarter(s); });
  fill("fill_decode_k16", 32 * 16, [](unsigned s) { return fill_chunk_decode_k<16>(s); });
  fill("fill_decode_k8", 32 * 8, [](unsigned s) { return fill_chunk_decode_k<8>(s); });
  fill("fill_decode16", 32 * 16, [](unsigned s) { return fill_chunk_decode<16>(s); });
  fill("fill_decode8", 32 * 8, [](unsigned s) { return fill_chunk_decode<8>(s); });
  // reads, indexed [first argument][second argument][lane]
  key("prefill_k16");
  list(8, [](int s) { lanes(k16<16>, s, 0); });
  key("prefill_k8");
  list(4, [](int s) { lanes(k16<8>, s, 0); });
  key("prefill_vt16");
  list(2, [](int hf) { list(4, [&](int t) { lanes(vt16<16>, hf, t); }); });
  key("prefill_vt8");
  list(2, [](int hf) { list(2, [&](int t) { lanes(vt16<8>, hf, t); }); });
  key("fp8_ka");
  list(2, [](int s) { list(2, [&](int c) { lanes(ka8, s, c); }); });
  key("fp8_kb");
  list(2, [](int c) { lanes(kb8, c, 0); });
  key("fp8_vt");
  list(4, [](int t) { lanes(vt8, t, 0); });
  key("decode_k16");
  list(4, [](int s) { lanes(dk<16>, s, 0); });
  key("decode_k8");
  list(2, [](int s) { lanes(dk<8>, s, 0); });
  key("decode_vt16");
  list(2, [](int hf) { list(8, [&](int t) { lanes(dvt<16>, hf, t); }); });
  key("decode_vt8");
  list(2, [](int hf) { list(4, [&](int t) { lanes(dvt<8>, hf, t); }); });
  std::printf("\n}\n");
  return 0;
}
