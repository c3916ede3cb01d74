// Host-only harness for the GGUF reader and definition compiler in
// decoder_gguf_quantized_amd/csrc/gguf.cpp, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_gguf_fuzz.py.  Arguments are model
// files, each parsed with the current definition text; "-d FILE" makes FILE's
// contents the definition text for the files after it ("-d -" returns to the
// built-in definition).  For each file qdec_gguf_config must return QDEC_OK
// or QDEC_REFUSED; a crash, an out-of-bounds read or undefined behaviour
// aborts the process.  The two library calls gguf.cpp makes outside itself
// are stubbed here.
#include <cstdio>
#include <cstring>
#include <fstream>
#include <sstream>
#include <string>

#include "../../include/qdec.h"

static std::string g_text;
void qdec_set_error_text(const std::string& s) { g_text = s; }

extern "C" int qdec_load_weights(const qdec_config*, const qdec_tensor*, int32_t, int32_t, int32_t, void*,
                                 qdec_model**) {
  return QDEC_REFUSED;
}

int main(int argc, char** argv) {
  int ok = 0, refused = 0;
  std::string def;
  bool have_def = false;
  for (int i = 1; i < argc; ++i) {
    if (std::strcmp(argv[i], "-d") == 0 && i + 1 < argc) {
      have_def = std::strcmp(argv[++i], "-") != 0;
      if (have_def) {
        std::ifstream f(argv[i], std::ios::binary);
        std::ostringstream ss;
        ss << f.rdbuf();
        def = ss.str();
      }
      continue;
    }
    qdec_config c;
    const int rc = qdec_gguf_config(argv[i], have_def ? def.c_str() : nullptr, &c);
    if (rc == QDEC_OK) ++ok;
    else if (rc == QDEC_REFUSED) ++refused;
    else {
      std::fprintf(stderr, "%s: status %d\n", argv[i], rc);
      return 3;
    }
  }
  std::printf("ok %d refused %d\n", ok, refused);
  return 0;
}
